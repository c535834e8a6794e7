// Replay attention backward for latent-KV heads on gfx950 (LongStraw study notes, §2-1 step 4 and
// §2-2; the latent-KV pages of the GLM run: the §3-1 overview table and §3-2 (1), (5)): Dqk = 576, Dv = 512, one kv head, V = the
// leading 512 dims of every K row. With P = exp(S scale - LSE), dP = dO V^T, Delta = rowsum(dO * O)
// and dS = P (dP - Delta):
//   dV_j += sum_rows P_rj dO_r,  dK_j += scale sum_rows dS_rj Q_r,  dQ_r = scale sum_j dS_rj K_j.
// MFMA 16x16x32 throughout. Transposed operands (K^T, Q^T, dO^T) are read from key- or row-major
// LDS tiles with ds_read_b64_tr_b16, so no dimension-major copies are packed.
//
// replay_bwd_dq_wide: query-tile owner (4 waves x 16 packed rows) with split-K over the prompt,
// like the forward. Per 32-key tile: S^T = K Q^T and dP^T = V dO^T share every K fragment read
// (V is K's leading dims), dS^T goes straight from the score registers into the B operand of
// dQ^T += K^T dS^T. Q and dO fragments (136 registers) and the dQ^T accumulators (144) stay in
// registers: one wave per SIMD.
//
// replay_bwd_dkdv_wide: key-tile owner (4 waves x 16 keys) looping over 32-row steps of the packed
// query rows. Per step: S = Q K^T and dP = dO V^T (A operands: rows of the staged Q / dO tiles, B:
// the wave's K fragments, which also serve as V fragments), P and dS as fp16 B operands, then
// dV^T += dO^T P and dK^T += Q^T dS. All four products run in fp16 on operands scaled by powers of
// two (Q, dO, K, and 2^15 P, dS) so that the fp32 accumulators of the prompt keys keep a relative
// error near 2^-12 per term; the scales come from a maxima pass over this call's inputs.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 lds_h128(const char* base, int off) { return lds_h128_at(base, off); }
__device__ __forceinline__ f16x8 join_tr_h(const s16x4& a, const s16x4& b) {
  return __builtin_bit_cast(f16x8, join_tr(a, b));
}

// LDS tiles of 576-dim rows (1152 B, 72 chunks) and of 512-dim rows (1024 B, 64 chunks): logical
// chunk c of row r sits at c ^ swz72(r) (low three bits) / c ^ swz64(r) (low four bits). Two read
// patterns hit them: interleaved-row fragment reads (16 bytes per lane, rows 8a + b and 8a + 4 + b,
// b < 4, one chunk per 16 lanes) and transposed reads (8 bytes per lane, rows 8q + 4u + e, e < 4,
// 32 bytes per row). Both swizzles were chosen by measuring LDS bank-conflict cycles
// (SQ_LDS_BANK_CONFLICT) for these patterns over linear swizzles of row bits 0, 1, 3, 4: each is a
// simplest one with no conflict cycles for either pattern at its pitch. Neither reads bit 2 (the
// two interleaved tiles, 4 rows apart, and the two halves of a transposed read share the swizzle).
__device__ __forceinline__ int swz72(int r) { return (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2); }
__device__ __forceinline__ int swz64(int r) { return (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2) | ((r & 1) << 3); }

constexpr int kD = kWideDqk, kDV = kWideDv;
constexpr int kRow72 = kD * 2, kRow64 = kDV * 2;

// ------------------------------------------------------------------ operand scales
__device__ __forceinline__ float pow2_fit_w(float x) {
  if (!(x > 0.0f)) return 1.0f;
  int e;
  (void)frexpf(x, &e);
  const int k = min(60, max(-60, 15 - e));
  return ldexpf(1.0f, k);
}

__device__ __forceinline__ void amax8(const u32x4& v, float& m) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    m = __builtin_elementwise_maximum(
        m, __builtin_elementwise_maximum(__builtin_fabsf(bf16_lo(v[q])), __builtin_fabsf(bf16_hi(v[q]))));
}
__device__ __forceinline__ float sq8(const u32x4& v) {
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) s = __builtin_fmaf(bf16_lo(v[q]), bf16_lo(v[q]), __builtin_fmaf(bf16_hi(v[q]), bf16_hi(v[q]), s));
  return s;
}

// Per block: {max |dO|, max row norm of dO, max |Q|, max row norm of V (the leading 512 dims of the
// K rows), max |K|}. A 512-dim row is one wave (16 bytes per lane); the K rows' last 64 dims are
// read by lanes 0-7.
__global__ __launch_bounds__(256) void wide_scale_partials(ScaleArgs a, const uint16_t* Kp, const uint16_t* Ks,
                                                           int64_t ldk) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  float v[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t nr = a.T * a.Hq;
  for (int64_t r = wave; r < nr; r += nwaves) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(a.dO + r * kDV + lane * 8);
    amax8(x, v[0]);
    v[1] = __builtin_elementwise_maximum(v[1], __builtin_sqrtf(wave_sum(sq8(x))));
    const u32x4 y = *reinterpret_cast<const u32x4*>(a.Q + r * kD + lane * 8);
    amax8(y, v[2]);
    if (lane < 8) amax8(*reinterpret_cast<const u32x4*>(a.Q + r * kD + 512 + lane * 8), v[2]);
  }
  for (int64_t r = wave; r < a.P + a.Tk; r += nwaves) {
    const uint16_t* row = r < a.P ? Kp + r * ldk : Ks + (r - a.P) * ldk;
    const u32x4 x = *reinterpret_cast<const u32x4*>(row + lane * 8);
    amax8(x, v[4]);
    v[3] = __builtin_elementwise_maximum(v[3], __builtin_sqrtf(wave_sum(sq8(x))));
    if (lane < 8) amax8(*reinterpret_cast<const u32x4*>(row + 512 + lane * 8), v[4]);
  }
  __shared__ float red[5][4];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const float x = wave_max(v[i]);
    if (lane == 0) red[i][threadIdx.x >> 6] = x;
  }
  __syncthreads();
  if (threadIdx.x < 5) {
    const int i = threadIdx.x;
    a.partial[blockIdx.x * 8 + i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(red[i][0], red[i][1]),
                                                                  __builtin_elementwise_maximum(red[i][2], red[i][3]));
  }
}

__global__ __launch_bounds__(256) void wide_scale_final(ScaleArgs a) {
  __shared__ float red[5][4];
  float v[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  for (int b = threadIdx.x; b < kScaleBlocks; b += 256)
#pragma unroll
    for (int i = 0; i < 5; ++i) v[i] = __builtin_elementwise_maximum(v[i], a.partial[b * 8 + i]);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const float x = wave_max(v[i]);
    if ((threadIdx.x & 63) == 0) red[i][threadIdx.x >> 6] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float m[5];
#pragma unroll
    for (int i = 0; i < 5; ++i)
      m[i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(red[i][0], red[i][1]),
                                           __builtin_elementwise_maximum(red[i][2], red[i][3]));
    a.scales[0] = pow2_fit_w(m[0]);
    a.scales[1] = pow2_fit_w(m[2]);
    // |2^15 P (dP - Delta)| <= 2^15 * 2 * max|dO_r| * max|V_j|: scale that bound down to 2^15
    a.scales[2] = pow2_fit_w(2.0f * m[1] * m[3]) * 0x1p-15f;
    a.scales[3] = pow2_fit_w(m[4]);
  }
}

// ------------------------------------------------------------------ dQ (query owner, split-K)
struct WideDqCfg {
  static constexpr int NW = 4;
  static constexpr int BM = NW * 16;
  static_assert(BM == kQTileDqWide, "dQ tile must match the plan");
  static constexpr int BN = 32;
  static constexpr int STAGE = BN * kRow72;
  static constexpr int NSTAGE = 4;
  static constexpr int NP = STAGE / 1024;
  static constexpr int PPW = NP / NW;
  static_assert(NP % NW == 0, "pieces split evenly over the waves");
  static constexpr int KS = kD / 32;   // score k-steps
  static constexpr int VS = kDV / 32;  // dP k-steps (the K fragments' leading 16)
  static constexpr int KT = kD / 16;   // 16-dim tiles of dQ^T
};

__global__ __launch_bounds__(64 * WideDqCfg::NW, 1) void replay_bwd_dq_wide(BwdArgs a) {
  using C = WideDqCfg;
  // one LDS array per ring stage (reads of one stage never wait for loads into another)
  __shared__ __attribute__((aligned(1024))) char sm0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sm1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sm2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sm3[C::STAGE];
  static_assert(C::NSTAGE == 4, "one array per stage");
  char* const stg[4] = {sm0, sm1, sm2, sm3};

  const AttnGeom& G = a.geo;
  const int W = a.qtiles * a.splits;
  const int per_xcd = (W + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= W) return;
  const int sp = w / a.qtiles;
  const int qt = w - sp * a.qtiles;
  int ri = 0;
  while (qt >= a.tile0[ri + 1]) ++ri;
  const int tokb = G.tok0[ri];
  const int R = G.tok0[ri + 1] - tokb;
  const int ktokb = G.ktok0[ri];
  const int Rk = G.ktok0[ri + 1] - ktokb;
  const int qo = Rk - R;
  const int g = G.g;
  const int M = R * g;
  const int m0 = (qt - a.tile0[ri]) * C::BM;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int i16 = lane & 15;
  const int q4 = lane >> 4;

  const int mrow = m0 + wv * 16 + i16;
  const bool rvalid = mrow < M;
  const int trow = rvalid ? mrow / g : 0;
  const int hq = rvalid ? mrow - trow * g : 0;
  const int64_t tok = tokb + trow;
  bf16x8 qf[C::KS], of[C::VS];
  {
    const uint16_t* qrow = G.Q + (tok * G.Hq + hq) * kD + q4 * 8;
    const uint16_t* orow = a.dO + (tok * G.Hq + hq) * kDV + q4 * 8;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qf[s] = rvalid ? ld_bf16x8(qrow + s * 32) : zero_bf16x8();
#pragma unroll
    for (int s = 0; s < C::VS; ++s) of[s] = rvalid ? ld_bf16x8(orow + s * 32) : zero_bf16x8();
  }
  // 2^x form: P = exp2(S scale log2 e - LSE log2 e); rows past the tile give P = 0
  const float lrow = rvalid ? a.lse[(int64_t)hq * G.T + tok] * kLog2e : INFINITY;
  const float drow = rvalid ? a.delta[(int64_t)hq * G.T + tok] : 0.0f;

  // fragment offsets (see the forward kernel: interleaved score tiles, transposed K^T reads)
  const int key_a = 8 * (i16 >> 2) + (i16 & 3);
  int kb[2];
#pragma unroll
  for (int s0 = 0; s0 < 2; ++s0) kb[s0] = key_a * kRow72 + (((4 * s0 + q4) ^ swz72(key_a)) << 4);
  const int key_t = 8 * q4 + (i16 >> 2);
  int tb[4];
  {
    const int b0 = key_t * kRow72 + ((((i16 >> 1) & 1) ^ swz72(key_t)) << 4) + ((i16 & 1) << 3);
#pragma unroll
    for (int d0 = 0; d0 < 4; ++d0) tb[d0] = b0 ^ (d0 << 5);
  }

  const int pkey0 = sp * a.ptiles_per_split * 64;
  const int pkey1 = min(G.P, pkey0 + a.ptiles_per_split * 64);
  const int nps = pkey1 > pkey0 ? (pkey1 - pkey0 + C::BN - 1) / C::BN : 0;
  const int t_lo = m0 / g + qo;
  const int t_hi = (min(M, m0 + C::BM) - 1) / g + qo;
  const int nss = (sp == a.splits - 1) ? t_hi / C::BN + 1 : 0;
  const int nit = nps + nss;

  const char* const kp0 = reinterpret_cast<const char*>(G.Kp);
  const char* const ks0 = reinterpret_cast<const char*>(G.Ks + (int64_t)ktokb * G.ldk);
  const int64_t kp_end = ((int64_t)(G.P - 1) * G.ldk + kD) * 2;
  const int64_t ks_end = ((int64_t)(G.Tk - 1 - ktokb) * G.ldk + kD) * 2;
  const int64_t ldk2 = G.ldk * 2;
  auto issue = [&](int u, auto jc) {
    const int uu = min(u, nit - 1);
    const bool pr = uu < nps;
    const int key0 = pr ? pkey0 + uu * C::BN : (uu - nps) * C::BN;
    const int64_t ko = key0 * ldk2;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc((pr ? kp0 : ks0) + ko, (pr ? kp_end : ks_end) - ko);
    char* dst = stg[decltype(jc)::value];
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < C::PPW; ++k) {
      const int pc = wv + C::NW * k;
      const int unit = pc * 64 + ln;
      const int row = unit / 72;
      const int c = (unit - row * 72) ^ swz72(row);
      lds_dma16_buf(rs, (uint32_t)(row * ldk2 + (c << 4)), dst + pc * 1024);
    }
  };

  f32x4 dq[C::KT];
#pragma unroll
  for (int d = 0; d < C::KT; ++d) dq[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c2 = G.scale_log2;

  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;
  if (nit > 0) {
    issue(0, J0{});
    issue(1, J1{});
    issue(2, J2{});
  }
  // One tile (the ring runs in whole rounds of four; tiles past the last are fully masked).
  auto tile = [&](int u, auto jc) {
    constexpr int J = decltype(jc)::value;
    wait_vmem_le<2 * C::PPW>();
    wait_lds();
    bare_barrier();
    issue(u + 3, std::integral_constant<int, (J + 3) % 4>{});
    const char* sb = stg[J];
    // Run A: S^T and dP^T. Every fragment read is written out first; the schedule below issues the
    // reads of k-step s + 2 right after the MFMAs of step s, so LDS latency hides under the MFMAs.
    bf16x8 k0[C::KS], k1[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const int off = kb[s & 1] + 128 * (s >> 1);
      k0[s] = lds_b128_as(sb, off);
      k1[s] = lds_b128_as(sb, off + 4 * kRow72);
    }
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      st[0] = mfma16(k0[s], qf[s], st[0]);
      st[1] = mfma16(k1[s], qf[s], st[1]);
      if (s < C::VS) {
        dp[0] = mfma16(k0[s], of[s], dp[0]);
        dp[1] = mfma16(k1[s], of[s], dp[1]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      if (s < C::VS) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      else __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (s + 2 < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // first K^T fragments of run B, in flight during the dS arithmetic
    constexpr int LB = 4;
    s16x4 t0[C::KT], t1[C::KT];
    auto rd_t = [&](int d) {
      const int off = tb[d & 3] + 128 * (d >> 2);
      t0[d] = lds_tr_as(sb, off);
      t1[d] = lds_tr_as(sb, off + 4 * kRow72);
    };
#pragma unroll
    for (int d = 0; d < LB; ++d) rd_t(d);
    __builtin_amdgcn_sched_barrier(0);
    const bool live = u < nit;
    const bool pr = u < nps;
    const int key0 = pr ? pkey0 + u * C::BN : (u - nps) * C::BN;
    const int nvalid = min(C::BN, (pr ? G.P : Rk) - key0);
    const bool causal = !pr && (key0 + C::BN - 1 > t_lo);
    if (__builtin_expect(!live || causal || nvalid < C::BN, 0)) {
      asm volatile("");
      const int lim = (live ? min(nvalid, causal ? trow + qo - key0 + 1 : nvalid) : 0) - 8 * q4;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[h][r] = (4 * h + r) < lim ? st[h][r] : -INFINITY;
    }
    bf16x8 ds;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(__builtin_fmaf(st[h][r], c2, -lrow));
        ds[4 * h + r] = (__bf16)(p * (dp[h][r] - drow));
      }
    __builtin_amdgcn_sched_barrier(0);
    // Run B: dQ^T += K^T dS^T, the reads of fragment d + LB following the MFMA of fragment d
#pragma unroll
    for (int d = LB; d < C::KT; ++d) rd_t(d);
#pragma unroll
    for (int d = 0; d < C::KT; ++d) dq[d] = mfma16(join_tr(t0[d], t1[d]), ds, dq[d]);
#pragma unroll
    for (int d = 0; d < C::KT; ++d) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (d + LB < C::KT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int u0 = 0; u0 < nit; u0 += 4) {
    tile(u0, J0{});
    tile(u0 + 1, J1{});
    tile(u0 + 2, J2{});
    tile(u0 + 3, J3{});
  }
  wait_vmem();
  if (!rvalid) return;
  if (a.splits == 1) {
    uint16_t* dst = a.dQ + (tok * G.Hq + hq) * kD + 4 * q4;
    const float sc = G.scale;
#pragma unroll
    for (int d = 0; d < C::KT; ++d) {
      const u32x2 v = {pack_bf16x2(dq[d][0] * sc, dq[d][1] * sc), pack_bf16x2(dq[d][2] * sc, dq[d][3] * sc)};
      *reinterpret_cast<u32x2*>(dst + 16 * d) = v;
    }
  } else {
    float* dst = a.dq_part + (((int64_t)sp * G.T + tok) * G.Hq + hq) * kD + 4 * q4;
#pragma unroll
    for (int d = 0; d < C::KT; ++d) *reinterpret_cast<f32x4*>(dst + 16 * d) = dq[d];
  }
}

// ------------------------------------------------------------------ dK / dV (key owner)
struct WideKvCfg {
  static constexpr int NW = 4;
  static constexpr int BN = NW * 16;            // keys per workgroup
  static_assert(BN == kDKTileWide, "dK/dV tile must match the plan");
  static constexpr int BR = 32;                 // packed query rows per step
  static constexpr int QBYTES = BR * kRow72;    // fp16 Q rows
  static constexpr int OBYTES = BR * kRow64;    // fp16 dO rows
  static constexpr int OFF_O = QBYTES;
  static constexpr int OFF_RS = QBYTES + OBYTES;  // one 1 KB row-statistics piece per wave
  static constexpr int STAGE = OFF_RS + NW * 1024;
  static constexpr int NSTAGE = 2;
  static constexpr int QP = QBYTES / 1024, OP = OBYTES / 1024;
  static_assert(QP % NW == 0 && OP % NW == 0, "pieces split evenly over the waves");
  static constexpr int PPW = QP / NW + OP / NW + 1;
  static constexpr int KS = kD / 32, VS = kDV / 32;
  static constexpr int KT = kD / 16, VT = kDV / 16;
};

template <bool PROMPT>
__global__ __launch_bounds__(64 * WideKvCfg::NW, 1) void replay_bwd_dkdv_wide(BwdArgs a) {
  using C = WideKvCfg;
  // one LDS array per ring stage (reads of one stage never wait for loads into the other)
  __shared__ __attribute__((aligned(1024))) char sm0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sm1[C::STAGE];
  static_assert(C::NSTAGE == 2, "one array per stage");
  char* const stg[2] = {sm0, sm1};

  const AttnGeom& G = a.geo;
  const int nk = PROMPT ? a.ktiles_prompt : a.ktile0[G.n_resp];
  const int per_xcd = (nk + 7) >> 3;
  const int kt = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (kt >= nk) return;
  const int g = G.g;

  int key0, nkeys, tokb = 0, R = 0, ktokb = 0, qo = 0, row_begin, row_end;
  if (PROMPT) {
    key0 = kt * C::BN;
    nkeys = min(C::BN, G.P - key0);
    row_begin = 0;
    row_end = G.T * g;
  } else {
    int ri = 0;
    while (kt >= a.ktile0[ri + 1]) ++ri;
    tokb = G.tok0[ri];
    R = G.tok0[ri + 1] - tokb;
    ktokb = G.ktok0[ri];
    const int Rk = G.ktok0[ri + 1] - ktokb;
    qo = Rk - R;
    key0 = (kt - a.ktile0[ri]) * C::BN;
    nkeys = min(C::BN, Rk - key0);
    // the first row that sees key key0 sits at key position key0; rows of other responses in the
    // first step are masked below
    row_begin = ((tokb + max(0, key0 - qo)) * g) & ~(C::BR - 1);
    row_end = (tokb + R) * g;
  }
  const int nsteps = row_end > row_begin ? (row_end - row_begin + C::BR - 1) / C::BR : 0;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int i16 = lane & 15;
  const int q4 = lane >> 4;
  const int mykey = wv * 16 + i16;
  const bool kvalid = mykey < nkeys;

  // K fragments of this wave's 16 keys as fp16 (K * s_K): B operands of S = Q K^T (k-steps 0-17)
  // and of dP = dO V^T (k-steps 0-15, V being K's leading 512 dims); kept in AGPRs
  const float sK = a.scales[3];
  f16x8 kf[C::KS];
  {
    const uint16_t* kr = PROMPT ? G.Kp + (int64_t)(key0 + mykey) * G.ldk
                                : G.Ks + (int64_t)(ktokb + key0 + mykey) * G.ldk;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 v = kvalid ? *reinterpret_cast<const u32x4*>(kr + s * 32 + q4 * 8) : u32x4{0u, 0u, 0u, 0u};
      f16x8 h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[2 * q] = (_Float16)(bf16_lo(v[q]) * sK);
        h[2 * q + 1] = (_Float16)(bf16_hi(v[q]) * sK);
      }
      kf[s] = h;
      asm volatile("" : "+a"(kf[s]));
    }
  }
  const float sdO = a.scales[0], sQ = a.scales[1], sdS = a.scales[2];
  const float cS = G.scale_log2 / (sQ * sK);  // S * scale log2 e from the scaled product
  const float cP = sdS / (sdO * sK);           // dP * s_dS from the scaled product

  f32x4 dk[C::KT], dv[C::VT];
#pragma unroll
  for (int d = 0; d < C::KT; ++d) dk[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < C::VT; ++d) dv[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Row fragments: score tile h row i is step row 8 (i / 4) + 4 h + i % 4 (so that lane group q
  // of either tile holds rows 8q .. 8q + 7: the k index of the fp16 B operands P and dS).
  const int row_a = 8 * (i16 >> 2) + (i16 & 3);
  int qb[2], ob[4];
#pragma unroll
  for (int s0 = 0; s0 < 2; ++s0) qb[s0] = row_a * kRow72 + (((4 * s0 + q4) ^ swz72(row_a)) << 4);
  // 64-chunk rows: (4 s + q4) ^ f = 16 (s / 4) + ((4 (s % 4) + q4) ^ f), f < 16
#pragma unroll
  for (int s0 = 0; s0 < 4; ++s0) ob[s0] = C::OFF_O + row_a * kRow64 + (((4 * s0 + q4) ^ swz64(row_a)) << 4);
  // transposed reads: lane j of group q addresses row 8q + 4u + j / 4, dims 16 d + 4 (j % 4)
  const int row_t = 8 * q4 + (i16 >> 2);
  int qtb[4];
  {
    const int b0 = row_t * kRow72 + ((((i16 >> 1) & 1) ^ swz72(row_t)) << 4) + ((i16 & 1) << 3);
#pragma unroll
    for (int d0 = 0; d0 < 4; ++d0) qtb[d0] = b0 ^ (d0 << 5);
  }
  // 64-chunk rows: physical chunk (2d) ^ X with X = ((j >> 1) & 1) ^ swz64(row) (swz64 is equal for
  // the four rows j / 4 = 0..3 XOR-ed into bits 0-1 and the group bits 2-3), so offset = otb ^ 32 d
  const int otb = C::OFF_O + row_t * kRow64 + ((((i16 >> 1) & 1) ^ swz64(row_t)) << 4) + ((i16 & 1) << 3);

  // direct loads of step n (rows row_begin + 32 n ..): Q pieces, dO pieces, and every wave's own
  // row-statistics piece (rows from the step's first, 128 of them; only the first 32 are read)
  const char* const qsrc = reinterpret_cast<const char*>(a.Qr);
  const char* const osrc = reinterpret_cast<const char*>(a.dOr);
  const char* const rsrc = reinterpret_cast<const char*>(a.rowstat);
  const int64_t mpad = a.mpad;
  auto issue = [&](int n, auto jc) {
    const int nn = min(n, nsteps - 1);
    const int64_t m0 = row_begin + (int64_t)nn * C::BR;
    const __amdgpu_buffer_rsrc_t rq = buf_rsrc(qsrc + m0 * kRow72, (mpad - m0) * kRow72);
    const __amdgpu_buffer_rsrc_t ro = buf_rsrc(osrc + m0 * kRow64, (mpad - m0) * kRow64);
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(rsrc + m0 * 8, (mpad - m0) * 8);
    char* dst = stg[decltype(jc)::value];
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < C::QP / C::NW; ++k) {
      const int pc = wv + C::NW * k;
      const int unit = pc * 64 + ln;
      const int row = unit / 72;
      const int c = (unit - row * 72) ^ swz72(row);
      lds_dma16_buf(rq, (uint32_t)(row * kRow72 + (c << 4)), dst + pc * 1024);
    }
#pragma unroll
    for (int k = 0; k < C::OP / C::NW; ++k) {
      const int pc = wv + C::NW * k;
      const int unit = pc * 64 + ln;
      const int row = unit >> 6;
      const int c = (unit & 63) ^ swz64(row);
      lds_dma16_buf(ro, (uint32_t)(row * kRow64 + (c << 4)), dst + C::OFF_O + pc * 1024);
    }
    lds_dma16_buf(rr, (uint32_t)(ln * 16), dst + C::OFF_RS + wv * 1024);
  };

  const int key_local = key0 + mykey;  // (response keys: position within the response)
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  if (nsteps > 0) issue(0, J0{});
  // One 32-row step (the ring runs in whole rounds of two; a step past the last adds nothing).
  // Fragment reads are written out first and scheduled a fixed distance ahead of their MFMAs.
  constexpr int LB = 4;  // read-ahead (fragments) of the dV / dK run
  auto step = [&](int n, auto jc) {
    constexpr int J = decltype(jc)::value;
    wait_vmem_le<0>();
    wait_lds();
    bare_barrier();  // step n landed for all waves; step n - 1 is no longer read
    issue(n + 1, std::integral_constant<int, (J + 1) % 2>{});
    const char* sb = stg[J];
    // Run A: S = Q K^T and dP = dO V^T; the reads of k-step s + 1 follow the MFMAs of step s
    f16x8 qa[C::KS], qz[C::KS], oa[C::VS], oz[C::VS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const int off = qb[s & 1] + 128 * (s >> 1);
      qa[s] = lds_h128_as(sb, off);
      qz[s] = lds_h128_as(sb, off + 4 * kRow72);
      if (s < C::VS) {
        const int oo = ob[s & 3] + 256 * (s >> 2);
        oa[s] = lds_h128_as(sb, oo);
        oz[s] = lds_h128_as(sb, oo + 4 * kRow64);
      }
    }
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      st[0] = mfma16h(qa[s], kf[s], st[0]);
      st[1] = mfma16h(qz[s], kf[s], st[1]);
      if (s < C::VS) {
        dp[0] = mfma16h(oa[s], kf[s], dp[0]);
        dp[1] = mfma16h(oz[s], kf[s], dp[1]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      if (s < C::VS) __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      else __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (s + 1 < C::VS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      else if (s + 1 < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // row statistics of this lane's rows 8 q4 .. 8 q4 + 7, and the first fragments of run B
    f32x4 sv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) sv[k] = lds_f32x4_as(sb, C::OFF_RS + wv * 1024 + q4 * 64 + 16 * k);
    s16x4 ta[C::VT + C::KT], tz[C::VT + C::KT];  // dO^T fragments, then Q^T fragments
    auto rd_t = [&](int i) {
      const int off = i < C::VT ? (otb ^ (i << 5)) : qtb[(i - C::VT) & 3] + 128 * ((i - C::VT) >> 2);
      const int du = i < C::VT ? 4 * kRow64 : 4 * kRow72;
      ta[i] = lds_tr_as(sb, off);
      tz[i] = lds_tr_as(sb, off + du);
    };
#pragma unroll
    for (int i = 0; i < LB; ++i) rd_t(i);
    __builtin_amdgcn_sched_barrier(0);
    // this lane: key mykey, step rows 8 q4 + e (e = 4 h + r); statistics {LSE log2 e - 15, Delta s_dS}
    const bool live = n < nsteps;
    float pe[8], de[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * h + r;
        const float lr = sv[e >> 1][2 * (e & 1)], dr = sv[e >> 1][2 * (e & 1) + 1];
        pe[e] = fast_exp2(__builtin_fmaf(st[h][r], cS, -lr));  // 2^15 P
        de[e] = pe[e] * __builtin_fmaf(dp[h][r], cP, -dr);     // 2^15 P (dP - Delta) s_dS
      }
    if (!PROMPT) {
      // causal keys of one response: row (token t of the response) sees key positions <= t + qo
      const int mb = row_begin + n * C::BR + 8 * q4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = (mb + e) / g - tokb;
        const bool vis = t >= 0 && t < R && key_local <= t + qo;
        pe[e] = vis ? pe[e] : 0.0f;
        de[e] = vis ? de[e] : 0.0f;
      }
    }
    f16x8 pb, db;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[e] = (_Float16)(live ? pe[e] : 0.0f);
      db[e] = (_Float16)(live ? de[e] : 0.0f);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Run B: dV^T += dO^T P, then dK^T += Q^T dS (transposed fragments of the staged rows); the
    // reads of fragment i + LB follow the MFMA of fragment i
#pragma unroll
    for (int i = LB; i < C::VT + C::KT; ++i) rd_t(i);
#pragma unroll
    for (int d = 0; d < C::VT; ++d) dv[d] = mfma16h(join_tr_h(ta[d], tz[d]), pb, dv[d]);
#pragma unroll
    for (int d = 0; d < C::KT; ++d) dk[d] = mfma16h(join_tr_h(ta[C::VT + d], tz[C::VT + d]), db, dk[d]);
#pragma unroll
    for (int i = 0; i < C::VT + C::KT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + LB < C::VT + C::KT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int n0 = 0; n0 < nsteps; n0 += 2) {
    step(n0, J0{});
    step(n0 + 1, J1{});
  }
  wait_vmem();
  if (!kvalid) return;

  // lane: key mykey, dims 16 d + 4 q4 .. +3
  const float fv = 1.0f / (32768.0f * sdO);
  const float sc = G.scale / (32768.0f * sdS * sQ);
  if (PROMPT) {
    float* dvr = a.dVp + (int64_t)(key0 + mykey) * kDV + 4 * q4;
    float* dkr = a.dKp + (int64_t)(key0 + mykey) * kD + 4 * q4;
#pragma unroll
    for (int d = 0; d < C::VT; ++d) {
      f32x4* p = reinterpret_cast<f32x4*>(dvr + 16 * d);
      *p = *p + dv[d] * fv;
    }
#pragma unroll
    for (int d = 0; d < C::KT; ++d) {
      f32x4* p = reinterpret_cast<f32x4*>(dkr + 16 * d);
      *p = *p + dk[d] * sc;
    }
  } else if (a.dKs_acc) {
    const int64_t tk = ktokb + key0 + mykey;
    float* dvr = a.dVs_acc + tk * kDV + 4 * q4;
    float* dkr = a.dKs_acc + tk * kD + 4 * q4;
#pragma unroll
    for (int d = 0; d < C::VT; ++d) {
      f32x4* p = reinterpret_cast<f32x4*>(dvr + 16 * d);
      *p = *p + dv[d] * fv;
    }
#pragma unroll
    for (int d = 0; d < C::KT; ++d) {
      f32x4* p = reinterpret_cast<f32x4*>(dkr + 16 * d);
      *p = *p + dk[d] * sc;
    }
  } else {
    const int64_t tk = ktokb + key0 + mykey;
    uint16_t* dvr = a.dVs + tk * kDV + 4 * q4;
    uint16_t* dkr = a.dKs + tk * kD + 4 * q4;
#pragma unroll
    for (int d = 0; d < C::VT; ++d) {
      const u32x2 v = {pack_bf16x2(dv[d][0] * fv, dv[d][1] * fv), pack_bf16x2(dv[d][2] * fv, dv[d][3] * fv)};
      *reinterpret_cast<u32x2*>(dvr + 16 * d) = v;
    }
#pragma unroll
    for (int d = 0; d < C::KT; ++d) {
      const u32x2 v = {pack_bf16x2(dk[d][0] * sc, dk[d][1] * sc), pack_bf16x2(dk[d][2] * sc, dk[d][3] * sc)};
      *reinterpret_cast<u32x2*>(dkr + 16 * d) = v;
    }
  }
}

}  // namespace

hipError_t launch_bwd_dq_wide(BwdArgs& a, hipStream_t st) {
  const long long W = (long long)a.qtiles * a.splits;
  if (W == 0) return hipSuccess;
  timer_mark(LS_KERNEL_DQ, st, false);
  hipLaunchKernelGGL(replay_bwd_dq_wide, dim3((unsigned)(((W + 7) / 8) * 8)), dim3(64 * WideDqCfg::NW), 0, st, a);
  timer_mark(LS_KERNEL_DQ, st, true);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_wide(BwdArgs& a, hipStream_t st) {
  const AttnGeom& G = a.geo;
  hipError_t e;
  ScaleArgs sa;
  sa.dO = a.dO;
  sa.Q = G.Q;
  sa.Vp = G.Vp;
  sa.Vs = G.Vs;
  sa.ldv = G.ldv;
  sa.T = G.T;
  sa.Tk = G.Tk;
  sa.P = G.P;
  sa.Hq = G.Hq;
  sa.Hkv = G.Hkv;
  sa.Dqk = kD;
  sa.Dv = kDV;
  sa.partial = a.scale_part;
  sa.scales = a.scales;
  hipLaunchKernelGGL(wide_scale_partials, dim3(kScaleBlocks), dim3(256), 0, st, sa, G.Kp, G.Ks, G.ldk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(wide_scale_final, dim3(1), dim3(256), 0, st, sa);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // packed query rows, row-major fp16: Q * s_Q and dO * s_dO; per-row statistics
  const int64_t M = (int64_t)G.T * G.g;
  PackArgs p;
  p.ld = (int64_t)G.Hq * kD;
  p.grp = G.g;
  p.gstride = kD;
  p.hstride = (int64_t)G.g * kD;
  p.dim = kD;
  p.heads = 1;
  p.nseg = 1;
  p.row0[0] = 0;
  p.n[0] = (int32_t)M;
  p.col0[0] = 0;
  p.out_ld = a.mpad;
  p.cols = a.mpad;
  p.src = G.Q;
  p.out = a.Qr;
  p.f16_scale = a.scales + 1;
  if ((e = launch_pack_rows(p, st)) != hipSuccess) return e;
  p.ld = (int64_t)G.Hq * kDV;
  p.gstride = kDV;
  p.hstride = (int64_t)G.g * kDV;
  p.dim = kDV;
  p.src = a.dO;
  p.out = a.dOr;
  p.f16_scale = a.scales + 0;
  if ((e = launch_pack_rows(p, st)) != hipSuccess) return e;
  RowStatArgs r;
  r.lse = a.lse;
  r.delta = a.delta;
  r.scales = a.scales;
  r.out = a.rowstat;
  r.T = G.T;
  r.Hq = G.Hq;
  r.g = G.g;
  r.Hkv = 1;
  r.M = M;
  r.mpad = a.mpad;
  if ((e = launch_pack_rowstats(r, st)) != hipSuccess) return e;

  if (a.ktiles_prompt > 0) {
    const long long W = a.ktiles_prompt;
    timer_mark(LS_KERNEL_DKDV_PROMPT, st, false);
    hipLaunchKernelGGL(replay_bwd_dkdv_wide<true>, dim3((unsigned)(((W + 7) / 8) * 8)), dim3(64 * WideKvCfg::NW), 0,
                       st, a);
    timer_mark(LS_KERNEL_DKDV_PROMPT, st, true);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const long long W = a.ktile0[G.n_resp];
  if (W > 0) {
    hipLaunchKernelGGL(replay_bwd_dkdv_wide<false>, dim3((unsigned)(((W + 7) / 8) * 8)), dim3(64 * WideKvCfg::NW), 0,
                       st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lsr
