// Replay attention forward on gfx950 (LongStraw study notes, §2-1 step 4 and §3-2 (2)/(4)):
// the queries of one response attend to all prompt keys and, causally, to the response's
// own keys.
//
// replay_fwd: one workgroup = 4 waves x 64 = 256 GQA-packed query rows of one kv head (one wave
// per SIMD), over the prompt key tiles of one split (plus, in the last split, the response's
// causal key tiles). Per 64-key tile, K (key-major) and V (dimension-major, packed by pack.hip)
// stream global -> LDS by direct DMA into a three-stage ring of XOR-swizzled tiles. Per 32-key
// block each wave computes S^T = K Q^T for its two 32-row blocks (MFMA 32x32x16 bf16; Q fragments
// stay in registers; every K fragment read from LDS feeds two MFMAs), an online softmax whose row
// statistics are lane-local (one query row per lane), and O^T += V^T P^T where P^T comes straight
// from the score accumulators and every V^T fragment is one 16-byte LDS read feeding two MFMAs.
// The softmax stabiliser is only moved when a row maximum exceeds it by more than 2^8 (in exp2
// units), so the O rescale is rare; probabilities stay <= 256, far inside fp32/bf16 range.
// Workgroup ids are mapped so that each XCD owns a contiguous run of (kv head, split) streams:
// concurrently resident query tiles sweep the same prompt K/V tiles, which are then fetched from
// HBM once per XCD and served to its CUs from L2.
//
// replay_fwd_merge: log-sum-exp merge of the split partials,
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

template <int D, int DV>
struct FwdCfg {
  static constexpr int RB = 2;                // 32-row blocks per wave
  static constexpr int BM = 4 * 32 * RB;      // packed query rows per workgroup
  static constexpr int BN = 64;               // keys per tile
  static constexpr int KCH = D / 8;           // 16-byte chunks per K row
  static constexpr int KROW = D * 2;          // bytes per K row in LDS
  static constexpr int VTROW = BN * 2;        // bytes per packed V^T row (one dim, 64 keys)
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = DV * VTROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int NSTAGE = 3;
  static constexpr int KINS = KBYTES / 1024 / 4;  // 1 KB direct loads per wave per tile
  static constexpr int VINS = VBYTES / 1024 / 4;
  static constexpr int KS = D / 16;           // MFMA k-steps over the head dim
  static constexpr int NB = DV / 32;          // 32-wide blocks of the value dim
  static constexpr float kStale = 8.0f;       // stabiliser slack (exp2 units)
};

__device__ __forceinline__ float max3f(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }

// max / sum of a value over lanes l and l ^ 32. The swap of two copies of v leaves, in each lane,
// the lane's own value in one result and its partner's in the other; combining the two results
// with a commutative operation gives both lanes the same bits.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int DV>
__global__ __launch_bounds__(256, 1) void replay_fwd(FwdArgs a) {
  using C = FwdCfg<D, DV>;
  __shared__ __attribute__((aligned(1024))) char smem[C::NSTAGE * C::STAGE];

  const AttnGeom& G = a.geo;
  const int W = a.qtiles * G.Hkv * a.splits;
  const int per_xcd = (W + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= W) return;
  const int strm = w / a.qtiles;
  const int qt = w - strm * a.qtiles;
  const int kvh = strm / a.splits;
  const int sp = strm - kvh * a.splits;
  int ri = 0;
  while (qt >= a.tile0[ri + 1]) ++ri;
  const int tokb = G.tok0[ri];
  const int R = G.tok0[ri + 1] - tokb;
  const int g = G.g;
  const int M = R * g;
  const int m0 = (qt - a.tile0[ri]) * C::BM;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  // query rows: block rb of wave wv holds packed rows m0 + 64 wv + 32 rb + (lane % 32)
  bool rvalid[C::RB];
  int trow[C::RB], hq[C::RB];
  bf16x8 qf[C::RB][C::KS];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const int mrow = m0 + wv * 32 * C::RB + rb * 32 + l32;
    rvalid[rb] = mrow < M;
    trow[rb] = rvalid[rb] ? mrow / g : 0;
    hq[rb] = kvh * g + (rvalid[rb] ? mrow - trow[rb] * g : 0);
    const uint16_t* qrow = G.Q + ((int64_t)(tokb + trow[rb]) * G.Hq + hq[rb]) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (rvalid[rb]) qf[rb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + ks * 16));
      else qf[rb][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      // Q fragments are only ever MFMA operands: keep them in AGPRs
      asm volatile("" : "+a"(qf[rb][ks]));
    }
  }

  // lane-constant LDS byte offsets within a stage (block and tile offsets are immediates)
  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = l32 * C::KROW + (((2 * ks + hl) ^ swz<C::KCH>(l32)) << 4);
  int voff[2][2];  // [32-key block][16-key half]: packed slots 32 kb + 16 h + 8 hl .. +7 of dim row l32
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) voff[kb][h] = C::KBYTES + l32 * C::VTROW + (((4 * kb + 2 * h + hl) ^ swz<8>(l32)) << 4);

  // key range: prompt tiles of this split, then (last split) the response's causal tiles
  const int pt0 = sp * a.ptiles_per_split;
  const int np = max(0, min(a.ptiles, pt0 + a.ptiles_per_split) - pt0);
  const int t_lo = m0 / g;
  const int t_hi = (min(M, m0 + C::BM) - 1) / g;
  const int ns = (sp == a.splits - 1) ? (t_hi / C::BN + 1) : 0;
  const int nit = np + ns;

  // Per-lane byte offsets of the direct loads within a full tile (32-bit, added to a wave-uniform
  // tile base): K rows are key-major (1024 / KROW rows per 1 KB instruction), packed V^T rows
  // are dimension-major (8 rows of 128 bytes per instruction).
  uint32_t kdo[C::KINS], vdo[C::VINS];
#pragma unroll
  for (int u = 0; u < C::KINS; ++u) {
    const int row = (wv * C::KINS + u) * (64 / C::KCH) + lane / C::KCH;
    kdo[u] = (uint32_t)(row * G.ldk * 2 + (((lane % C::KCH) ^ swz<C::KCH>(row)) << 4));
  }
#pragma unroll
  for (int u = 0; u < C::VINS; ++u) {
    const int row = (wv * C::VINS + u) * 8 + (lane >> 3);
    vdo[u] = (uint32_t)(row * a.ppad * 2 + (((lane & 7) ^ swz<8>(row)) << 4));
  }

  // global -> LDS for tile `it` into stage buffer `buf`
  auto issue_tile = [&](int it, char* buf) {
    if (it < np) {
      const int key0 = (pt0 + it) * C::BN;
      const int nvalid = min(C::BN, G.P - key0);
      const char* kb = reinterpret_cast<const char*>(G.Kp + (int64_t)key0 * G.ldk + kvh * D);
      const char* vb = reinterpret_cast<const char*>(a.VTp + (int64_t)kvh * DV * a.ppad + key0);
      if (nvalid == C::BN) {
#pragma unroll
        for (int u = 0; u < C::KINS; ++u) lds_dma16(kb + kdo[u], buf + (wv * C::KINS + u) * 1024);
#pragma unroll
        for (int u = 0; u < C::VINS; ++u) lds_dma16(vb + vdo[u], buf + C::KBYTES + (wv * C::VINS + u) * 1024);
        return;
      }
    }
    // ragged prompt tail or response keys: rows past the valid keys re-read the last valid row
    // (finite data, masked out of the softmax); packed V^T slots past the keys hold zeros
    const bool pr = it < np;
    const int key0 = pr ? (pt0 + it) * C::BN : (it - np) * C::BN;
    const int nvalid = min(C::BN, (pr ? G.P : R) - key0);
    const uint16_t* kb = pr ? G.Kp + (int64_t)key0 * G.ldk + kvh * D
                            : G.Ks + (int64_t)(tokb + key0) * G.ldk + kvh * D;
    const uint16_t* vb = pr ? a.VTp + (int64_t)kvh * DV * a.ppad + key0
                            : a.VTs + (int64_t)kvh * DV * a.tpad + a.spos[ri] + key0;
    const int64_t vld = pr ? a.ppad : a.tpad;
#pragma unroll
    for (int u = 0; u < C::KINS; ++u) {
      const int ins = wv * C::KINS + u;
      const int row = ins * (64 / C::KCH) + lane / C::KCH;
      const int c = (lane % C::KCH) ^ swz<C::KCH>(row);
      lds_dma16(kb + (int64_t)min(row, nvalid - 1) * G.ldk + c * 8, buf + ins * 1024);
    }
#pragma unroll
    for (int u = 0; u < C::VINS; ++u) {
      const int ins = wv * C::VINS + u;
      const int row = ins * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz<8>(row);
      lds_dma16(vb + (int64_t)row * vld + c * 8, buf + C::KBYTES + ins * 1024);
    }
  };

  f32x16 o[C::RB][C::NB];
  float mu[C::RB], l_run[C::RB];   // stabiliser (score * scale * log2 e) and row sum of this lane's keys
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    mu[rb] = -INFINITY;
    l_run[rb] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) o[rb][nb] = f32x16{};
  }
  const float c2 = G.scale_log2;

  // online softmax of one 32-row block (one query row per lane; the other half-wave holds the
  // row's other keys); returns the probabilities as the two bf16 B operands of the PV product
  auto softmax = [&](int rb, f32x16& st, bf16x8& p0, bf16x8& p1) {
    float mx = __builtin_elementwise_maximum(st[0], st[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, st[r]);
    mx = pair_max(mx) * c2;
    const bool move = mx > mu[rb] + C::kStale;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(move) != 0, 0)) {
      asm volatile("");  // rare: a real branch, never speculated into unconditional multiplies
      const float mnew = move ? mx : mu[rb];
      const float alpha = move ? fast_exp2(mu[rb] - mnew) : 1.0f;   // 0 on a row's first visible keys
      mu[rb] = mnew;
      l_run[rb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[rb][nb] *= alpha;
    }
    const float msub = mu[rb] == -INFINITY ? 0.0f : mu[rb];
    // the row sum is taken in fp32 (the LSE must hold to ~1e-6 even over a few keys)
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      st[r] = fast_exp2(__builtin_fmaf(st[r], c2, -msub));
      st[r + 1] = fast_exp2(__builtin_fmaf(st[r + 1], c2, -msub));
      ls0 += st[r];
      ls1 += st[r + 1];
    }
    l_run[rb] += ls0 + ls1;
    p0 = c_regs_to_bf16x8(st, 0);
    p1 = c_regs_to_bf16x8(st, 8);
  };

  auto compute = [&](const char* buf, bool masked, int key0, int nvalid, bool causal) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T for both row blocks; every K fragment feeds two MFMAs
      bf16x8 kf[C::KS];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) kf[ks] = lds_b128_at(buf, kb * 32 * C::KROW + koff[ks]);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 st[C::RB];
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        st[rb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) st[rb] = mfma32(kf[ks], qf[rb][ks], st[rb]);
      }
      // V^T fragments (one 16-byte read of packed slots each) arrive while the scores are formed
      bf16x8 vf[2][C::NB];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) vf[h][nb] = lds_b128_at(buf, nb * 32 * C::VTROW + voff[kb][h]);
      __builtin_amdgcn_sched_barrier(0);
      if (__builtin_expect(masked, 0)) {
        asm volatile("");  // keeps this a real (wave-uniform) branch instead of per-element selects
        // register r holds tile key kb*32 + 8(r/4) + 4hl + r%4; it is visible iff that key is below
        // nvalid and (causal tiles) key0 + key <= the row's token
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          const int lim = min(nvalid, causal ? trow[rb] - key0 + 1 : nvalid) - kb * 32 - 4 * hl;
#pragma unroll
          for (int r = 0; r < 16; ++r) st[rb][r] = (8 * (r >> 2) + (r & 3)) < lim ? st[rb][r] : -INFINITY;
        }
      }
      // row block 0's softmax runs under row block 1's score MFMAs, row block 1's under
      // row block 0's PV MFMAs
      bf16x8 pb[C::RB][2];
      softmax(0, st[0], pb[0][0], pb[0][1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) o[0][nb] = mfma32(vf[h][nb], pb[0][h], o[0][nb]);
      __builtin_amdgcn_sched_barrier(0);
      softmax(1, st[1], pb[1][0], pb[1][1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) o[1][nb] = mfma32(vf[h][nb], pb[1][h], o[1][nb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // three-stage ring: tile it+2 streams in while tile it is computed. Before computing tile it,
  // wait for this wave's loads of tile it (tile it+1's stay in flight), then a barrier makes every
  // wave's part visible and retires all reads of the stage refilled next (tile it-1's).
  char* const st0 = smem;
  char* const st1 = smem + C::STAGE;
  char* const st2 = smem + 2 * C::STAGE;
  constexpr int kPerTile = C::KINS + C::VINS;
  if (nit > 0) issue_tile(0, st0);
  if (nit > 1) issue_tile(1, st1);
  for (int it = 0; it < nit; it += 3) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int t = it + j;
      if (t >= nit) break;
      char* cur = j == 0 ? st0 : (j == 1 ? st1 : st2);
      char* nxt = j == 0 ? st2 : (j == 1 ? st0 : st1);
      if (t + 1 < nit) wait_vmem_le<kPerTile>();
      else wait_vmem();
      __syncthreads();
      if (t + 2 < nit) issue_tile(t + 2, nxt);
      const bool sfx = t >= np;
      const int key0 = sfx ? (t - np) * C::BN : (pt0 + t) * C::BN;
      const int nvalid = min(C::BN, (sfx ? R : G.P) - key0);
      const bool causal = sfx && (key0 + C::BN - 1 > t_lo);
      compute(cur, causal || nvalid < C::BN, key0, nvalid, causal);
    }
  }

#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const float l = pair_sum(l_run[rb]);
    if (!rvalid[rb]) continue;
    const int64_t tok = tokb + trow[rb];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float lse = l > 0.0f ? (mu[rb] + fast_log2(l)) * kLn2 : -INFINITY;
    if (a.splits == 1) {
      uint16_t* orow = a.O + (tok * G.Hq + hq[rb]) * DV + 4 * hl;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 v = {pack_bf16x2(o[rb][nb][4 * q] * inv, o[rb][nb][4 * q + 1] * inv),
                           pack_bf16x2(o[rb][nb][4 * q + 2] * inv, o[rb][nb][4 * q + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + nb * 32 + 8 * q) = v;
        }
      if (hl == 0) a.lse[(int64_t)hq[rb] * G.T + tok] = lse;
    } else {
      float* orow = a.o_part + (((int64_t)sp * G.T + tok) * G.Hq + hq[rb]) * DV + 4 * hl;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {o[rb][nb][4 * q] * inv, o[rb][nb][4 * q + 1] * inv, o[rb][nb][4 * q + 2] * inv,
                           o[rb][nb][4 * q + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + nb * 32 + 8 * q) = v;
        }
      if (hl == 0) a.lse_part[((int64_t)sp * G.Hq + hq[rb]) * G.T + tok] = lse;
    }
  }
}

template <int DV>
__global__ __launch_bounds__(256) void replay_fwd_merge(FwdArgs a) {
  const AttnGeom& G = a.geo;
  constexpr int CH = DV / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)G.T * G.Hq * CH;
  if (idx >= total) return;
  const int c = (int)(idx % CH);
  const int64_t th = idx / CH;
  const int h = (int)(th % G.Hq);
  const int64_t t = th / G.Hq;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s) mx = fmaxf(mx, a.lse_part[((int64_t)s * G.Hq + h) * G.T + t]);
  float den = 0.0f;
  for (int s = 0; s < a.splits; ++s) den += expf(a.lse_part[((int64_t)s * G.Hq + h) * G.T + t] - mx);
  const float lse = mx + logf(den);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) {
    const float wgt = expf(a.lse_part[((int64_t)s * G.Hq + h) * G.T + t] - lse);
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.o_part + (((int64_t)s * G.T + t) * G.Hq + h) * DV + 4 * c);
    acc += wgt * v;
  }
  const u32x2 ov = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  *reinterpret_cast<u32x2*>(a.O + (t * G.Hq + h) * DV + 4 * c) = ov;
  if (c == 0) a.lse[(int64_t)h * G.T + t] = lse;
}

template <int D, int DV>
hipError_t fwd_go(FwdArgs& a, hipStream_t st) {
  const long long W = (long long)a.qtiles * a.geo.Hkv * a.splits;
  if (W == 0) return hipSuccess;
  // dimension-major packed V of the prompt and of every response
  const AttnGeom& G = a.geo;
  if (G.P > 0) {
    PackArgs p;
    p.f16_scale = nullptr;
    p.src = G.Vp;
    p.ld = G.ldv;
    p.dim = DV;
    p.heads = G.Hkv;
    p.grp = 1;
    p.gstride = 0;
    p.hstride = DV;
    p.nseg = 1;
    p.row0[0] = 0;
    p.n[0] = G.P;
    p.col0[0] = 0;
    p.out = const_cast<uint16_t*>(a.VTp);
    p.out_ld = a.ppad;
    p.cols = a.ppad;
    hipError_t e = launch_pack_keys_t(p, st);
    if (e != hipSuccess) return e;
  }
  {
    PackArgs p;
    p.f16_scale = nullptr;
    p.src = G.Vs;
    p.ld = G.ldv;
    p.dim = DV;
    p.heads = G.Hkv;
    p.grp = 1;
    p.gstride = 0;
    p.hstride = DV;
    p.nseg = G.n_resp;
    for (int i = 0; i < G.n_resp; ++i) {
      p.row0[i] = G.tok0[i];
      p.n[i] = G.tok0[i + 1] - G.tok0[i];
      p.col0[i] = a.spos[i];
    }
    p.out = const_cast<uint16_t*>(a.VTs);
    p.out_ld = a.tpad;
    p.cols = a.tpad;
    hipError_t e = launch_pack_keys_t(p, st);
    if (e != hipSuccess) return e;
  }
  const long long per_xcd = (W + 7) / 8;
  timer_mark(LS_KERNEL_ATTN_FWD, st, false);
  hipLaunchKernelGGL((replay_fwd<D, DV>), dim3((unsigned)(per_xcd * 8)), dim3(256), 0, st, a);
  timer_mark(LS_KERNEL_ATTN_FWD, st, true);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const long long total = (long long)a.geo.T * a.geo.Hq * (DV / 4);
  hipLaunchKernelGGL((replay_fwd_merge<DV>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(FwdArgs& a, int Dqk, int Dv, hipStream_t st) {
  if (Dqk == 64 && Dv == 64) return fwd_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return fwd_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
