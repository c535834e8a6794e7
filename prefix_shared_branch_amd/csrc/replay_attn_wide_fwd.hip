// Replay attention forward for latent-KV heads on gfx950 (LongStraw study notes, §2-1 step 4 and
// §3-2 (2)/(4); the latent-KV pages of the GLM run: the §3-1 overview table and §3-2 (1), (5)): Dqk = 576, Dv = 512, one kv head, and
// V is the leading 512 dims of every K row (same rows, same row stride), so a single K tile in LDS
// serves both products.
//
// replay_fwd_wide: one workgroup = 8 waves x 16 = 128 GQA-packed query rows over the key tiles of
// one split (plus, in the last split, the response's causal keys), in 32-key tiles streamed
// global -> LDS by direct buffer loads into a four-stage ring. MFMA 16x16x32 bf16 throughout; per
// tile each wave computes
//   S^T = K Q^T    two 16-key score tiles whose keys are interleaved so that, after the softmax,
//                  lane group q of either tile holds keys 8q .. 8q + 7 of its row: exactly the
//                  B operand (P^T) of the next product, with no data movement;
//   O^T += V^T P^T the V^T fragments come from the key-major tile by transposed LDS reads
//                  (ds_read_b64_tr_b16), two per fragment.
// Q fragments (72 registers) and the O^T accumulators (128) stay in registers, so two waves share
// each SIMD and the hardware overlaps one wave's softmax with the other's MFMAs.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups holding one row's keys).
// Each swap leaves the lane's own value in one result and its partner's in the other; a
// commutative combination gives both partners the same bits.
__device__ __forceinline__ float quad_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct WideFwdCfg {
  static constexpr int D = kWideDqk, DV = kWideDv;
  static constexpr int NW = 8;                 // waves, two per SIMD
  static constexpr int BM = NW * 16;           // packed query rows per workgroup
  static_assert(BM == kQTileFwdWide, "forward tile must match the plan");
  static constexpr int BN = 32;                // keys per tile
  static constexpr int KROW = D * 2;           // bytes per K row
  static constexpr int STAGE = BN * KROW;      // 36 KB
  static constexpr int NSTAGE = 4;
  static constexpr int NP = STAGE / 1024;      // 1 KB direct-load pieces per tile
  static constexpr int PPW = 5;                // direct loads per wave per tile (see issue)
  static_assert(NP == 4 * NW + 4, "four pieces per wave, then one more for waves 0-3");
  static constexpr int KS = D / 32;            // k-steps of the score product
  static constexpr int DT = DV / 16;           // 16-dim tiles of O^T
  static constexpr float kStale = 8.0f;        // stabiliser slack (exp2 units)
};

// LDS K tile: row r (key) holds 72 chunks of 16 bytes; logical chunk c sits at c ^ wide_swz(r)
// (only the low three bits change, so a chunk stays in its group of eight). Two read patterns hit
// the tile: score-tile reads (16 bytes per lane, keys 8a + b and 8a + 4 + b, b < 4, one chunk per
// 16 lanes) and transposed reads (8 bytes per lane, keys 8q + 4u + e, e < 4, 32 bytes per key).
// With the 1152-byte pitch, this swizzle (bits 3 and 1 of the key into chunk bits 1 and 2) is the
// simplest one that measured zero LDS bank-conflict cycles for both patterns among all linear
// 3-bit swizzles of key bits 0, 1, 3, 4 (SQ_LDS_BANK_CONFLICT on gfx950). It ignores bit 2, so the
// two score tiles (keys 4 apart) and both halves of a transposed read share it.
__device__ __forceinline__ int wide_swz(int r) { return (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2); }

__global__ __launch_bounds__(64 * WideFwdCfg::NW, 1) void replay_fwd_wide(FwdArgs a) {
  using C = WideFwdCfg;
  // one LDS array per ring stage: the compiler then tells a stage's transposed reads apart from the
  // direct loads in flight into the other stages (and waits for none of them)
  __shared__ __attribute__((aligned(1024))) char sm0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sm1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sm2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sm3[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char sdummy[4 * 1024];
  static_assert(C::NSTAGE == 4, "one array per stage");
  char* const stg[4] = {sm0, sm1, sm2, sm3};

  const AttnGeom& G = a.geo;
  const int W = a.qtiles * a.splits;  // one kv head
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
  const int qo = Rk - R;  // query row t sits at key position t + qo
  const int g = G.g;
  const int M = R * g;
  const int m0 = (qt - a.tile0[ri]) * C::BM;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int i16 = lane & 15;
  const int q4 = lane >> 4;

  // query row of this lane (B operand column): packed row m0 + 16 wv + lane % 16
  const int mrow = m0 + wv * 16 + i16;
  const bool rvalid = mrow < M;
  const int trow = rvalid ? mrow / g : 0;
  const int hq = rvalid ? mrow - trow * g : 0;
  bf16x8 qf[C::KS];
  {
    const uint16_t* qrow = G.Q + ((int64_t)(tokb + trow) * G.Hq + hq) * C::D + q4 * 8;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) qf[s] = rvalid ? ld_bf16x8(qrow + s * 32) : zero_bf16x8();
  }

  // Score tile h (0, 1) row i is key 8 (i / 4) + 4 h + i % 4 of the 32-key tile; its k-step s
  // fragment is logical chunk 4 s + q4 of that row. With f = wide_swz(key) (equal for both tiles),
  // (4 s + q4) ^ f = 8 (s / 2) + ((4 (s % 2) + q4) ^ f), so two lane bases cover every k-step.
  const int key_a = 8 * (i16 >> 2) + (i16 & 3);
  int kb[2];
#pragma unroll
  for (int s0 = 0; s0 < 2; ++s0) kb[s0] = key_a * C::KROW + (((4 * s0 + q4) ^ wide_swz(key_a)) << 4);
  // Transposed V^T reads: lane j of group q addresses key 8q + 4u + j / 4, dims 16 d + 4 (j % 4) .. +3
  // and receives dims 16 d + j of keys 8q + 4u .. +3. Its chunk 2d + (j / 2) % 2 sits at
  // (2d) ^ X with X = ((j / 2) % 2) ^ wide_swz(row) (the swizzle does not depend on u), i.e. at byte
  // (32 d) ^ 16 X of the row: for d = 4 d' + d0 the offset is vb[d0] + 128 d' (+ 4 rows for u = 1).
  const int key_t = 8 * q4 + (i16 >> 2);
  int vb[4];
  {
    const int b0 = key_t * C::KROW + ((((i16 >> 1) & 1) ^ wide_swz(key_t)) << 4) + ((i16 & 1) << 3);
#pragma unroll
    for (int d0 = 0; d0 < 4; ++d0) vb[d0] = b0 ^ (d0 << 5);
  }

  // key range: 32-key tiles of this split's prompt keys, then (last split) the causal response keys
  const int pkey0 = sp * a.ptiles_per_split * 64;
  const int pkey1 = min(G.P, pkey0 + a.ptiles_per_split * 64);
  const int nps = pkey1 > pkey0 ? (pkey1 - pkey0 + C::BN - 1) / C::BN : 0;
  const int t_lo = m0 / g + qo;
  const int t_hi = (min(M, m0 + C::BM) - 1) / g + qo;
  const int nss = (sp == a.splits - 1) ? t_hi / C::BN + 1 : 0;
  const int nit = nps + nss;

  // global -> LDS: piece pc (1 KB) of a tile covers 16-byte units 64 pc .. 64 pc + 63 of the
  // key-major tile (72 units per row); waves 0-3 move pieces wv, wv + 4, ... Buffer resources end
  // with the key arrays, so rows past the last key read as zeros (masked out of the softmax).
  const char* const kp0 = reinterpret_cast<const char*>(G.Kp);
  const char* const ks0 = reinterpret_cast<const char*>(G.Ks + (int64_t)ktokb * G.ldk);
  const int64_t kp_end = ((int64_t)(G.P - 1) * G.ldk + C::D) * 2;
  const int64_t ks_end = ((int64_t)(G.Tk - 1 - ktokb) * G.ldk + C::D) * 2;
  const int64_t ldk2 = G.ldk * 2;
  auto issue = [&](int u, auto jc) {
    const int uu = min(u, nit - 1);  // past the last tile: reload it (keeps the wait counts fixed)
    const bool pr = uu < nps;
    const int key0 = pr ? pkey0 + uu * C::BN : (uu - nps) * C::BN;
    const int64_t ko = key0 * ldk2;
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc((pr ? kp0 : ks0) + ko, (pr ? kp_end : ks_end) - ko);
    char* dst = stg[decltype(jc)::value];
    int ln = lane;
    asm volatile("" : "+v"(ln));  // per-lane offsets recomputed per tile rather than pinned
#pragma unroll
    for (int k = 0; k < C::PPW; ++k) {
      // pieces wv, wv + 8, wv + 16, wv + 24, then 32 + wv for waves 0-3; waves 4-7 load the tile's
      // first kilobyte (just fetched by wave 0) into a scratch slot, so that every wave issues the
      // same number of loads per tile
      const bool real = k < C::PPW - 1 || wv < 4;
      const int pc = k < C::PPW - 1 ? wv + C::NW * k : C::NP - 4 + (wv & 3);
      const int unit = pc * 64 + ln;
      const int row = unit / 72;
      const int c = (unit - row * 72) ^ wide_swz(row);
      const uint32_t voff = real ? (uint32_t)(row * ldk2 + (c << 4)) : (uint32_t)(ln << 4);
      lds_dma16_buf(rs, voff, real ? dst + pc * 1024 : sdummy + (wv - 4) * 1024);
    }
  };

  f32x4 o[C::DT];
#pragma unroll
  for (int d = 0; d < C::DT; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mu = -INFINITY;  // stabiliser (score * scale * log2 e) of this lane's row
  float l_run = 0.0f;    // sum over this lane's keys
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
  // One tile: wait for its pieces, hand the stage of tile u - 1 to the loads of tile u + 3, then
  // S^T (run A), softmax, O^T += V^T P^T (run B). The reads of each run are written out first; the
  // schedule issues them a fixed distance ahead of the MFMAs that use them. Tiles past the last
  // (the ring runs in whole rounds of four) are fully masked and change nothing.
  constexpr int LA = 1, LB = 2;  // read-ahead distance in k-steps / dim tiles
  auto tile = [&](int u, auto jc) {
    constexpr int J = decltype(jc)::value;
    wait_vmem_le<2 * C::PPW>();  // this wave's pieces of tile u have landed
    wait_lds();
    bare_barrier();              // all pieces of tile u landed; tile u - 1 is no longer read
    issue(u + 3, std::integral_constant<int, (J + 3) % 4>{});
    const char* sb = stg[J];
    bf16x8 k0[C::KS], k1[C::KS];
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const int off = kb[s & 1] + 128 * (s >> 1);
      k0[s] = lds_b128_as(sb, off);
      k1[s] = lds_b128_as(sb, off + 4 * C::KROW);
    }
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      st[0] = mfma16(k0[s], qf[s], st[0]);
      st[1] = mfma16(k1[s], qf[s], st[1]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (s + LA < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    s16x4 t0[C::DT], t1[C::DT];
    auto rd_t = [&](int d) {
      const int off = vb[d & 3] + 128 * (d >> 2);
      t0[d] = lds_tr_as(sb, off);
      t1[d] = lds_tr_as(sb, off + 4 * C::KROW);
    };
#pragma unroll
    for (int d = 0; d < LB; ++d) rd_t(d);
    __builtin_amdgcn_sched_barrier(0);
    // softmax: this lane holds keys 8 q4 + 4 h + r (h = tile, r = register) of its row
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
    float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(st[0][0], st[0][1]),
                                             __builtin_elementwise_maximum(st[0][2], st[0][3]));
    mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(__builtin_elementwise_maximum(st[1][0], st[1][1]),
                                                                         __builtin_elementwise_maximum(st[1][2], st[1][3])));
    mx = quad_max(mx) * c2;
    const bool move = mx > mu + C::kStale;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(move) != 0, 0)) {
      asm volatile("");
      const float mnew = move ? mx : mu;
      const float alpha = move ? fast_exp2(mu - mnew) : 1.0f;  // 0 on a row's first visible keys
      mu = mnew;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DT; ++d) o[d] *= alpha;
    }
    const float msub = mu == -INFINITY ? 0.0f : mu;
    bf16x8 p;
    float ls = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(__builtin_fmaf(st[h][r], c2, -msub));
        ls += e;
        p[4 * h + r] = (__bf16)e;
      }
    l_run += ls;
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T over the tile's 32 keys
#pragma unroll
    for (int d = LB; d < C::DT; ++d) rd_t(d);
#pragma unroll
    for (int d = 0; d < C::DT; ++d) o[d] = mfma16(join_tr(t0[d], t1[d]), p, o[d]);
#pragma unroll
    for (int d = 0; d < C::DT; ++d) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (d + LB < C::DT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int u0 = 0; u0 < nit; u0 += 4) {
    tile(u0, J0{});
    tile(u0 + 1, J1{});
    tile(u0 + 2, J2{});
    tile(u0 + 3, J3{});
  }

  wait_vmem();  // the reloads issued past the last tile land before the workgroup's LDS is released
  const float l = quad_sum(l_run);
  if (!rvalid) return;
  const int64_t tok = tokb + trow;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float lse = l > 0.0f ? (mu + fast_log2(l)) * kLn2 : -INFINITY;
  // lane holds dims 16 d + 4 q4 .. +3 of its row
  if (a.splits == 1) {
    const int64_t off = (tok * G.Hq + hq) * C::DV + 4 * q4;
    uint16_t* orow = a.O + off;
#pragma unroll
    for (int d = 0; d < C::DT; ++d) {
      const f32x4 x = o[d] * inv;
      const u32x2 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *reinterpret_cast<u32x2*>(orow + 16 * d) = v;
      if (a.O_lo) {
        const u32x2 r = {pack_bf16x2_residual(x[0], x[1], v[0]), pack_bf16x2_residual(x[2], x[3], v[1])};
        *reinterpret_cast<u32x2*>(a.O_lo + off + 16 * d) = r;
      }
    }
    if (q4 == 0) a.lse[(int64_t)hq * G.T + tok] = lse;
  } else {
    float* orow = a.o_part + (((int64_t)sp * G.T + tok) * G.Hq + hq) * C::DV + 4 * q4;
#pragma unroll
    for (int d = 0; d < C::DT; ++d) *reinterpret_cast<f32x4*>(orow + 16 * d) = o[d] * inv;
    if (q4 == 0) a.lse_part[((int64_t)sp * G.Hq + hq) * G.T + tok] = lse;
  }
}

}  // namespace

hipError_t launch_attn_fwd_wide(FwdArgs& a, hipStream_t st) {
  const long long W = (long long)a.qtiles * a.splits;
  if (W == 0) return hipSuccess;
  const long long per_xcd = (W + 7) / 8;
  timer_mark(LS_KERNEL_ATTN_FWD, st, false);
  hipLaunchKernelGGL(replay_fwd_wide, dim3((unsigned)(per_xcd * 8)), dim3(64 * WideFwdCfg::NW), 0, st, a);
  timer_mark(LS_KERNEL_ATTN_FWD, st, true);
  return hipGetLastError();
}

}  // namespace lsr
