// Replay attention forward on gfx950 (LongStraw study notes, §2-1 step 4 and §3-2 (2)/(4)):
// the queries of one response attend to all prompt keys and, causally, to the response's
// own keys.
//
// replay_fwd: one workgroup = 4 waves x 64 = 256 GQA-packed query rows of one kv head, over
// the prompt key tiles of one split (plus, in the last split, the response's causal key
// tiles). 64-key K and V tiles stream global -> LDS by direct DMA (double-buffered, XOR-
// swizzled rows without padding). Per 32-key block each wave computes S^T = K Q^T for its two
// 32-row blocks (MFMA 32x32x16 bf16, Q fragments held in VGPRs, every K fragment read from LDS
// feeds two MFMAs), an online softmax whose row statistics are lane-local (one query row per
// lane; the O rescale is skipped when no row maximum moved), and O^T += V^T P^T with V^T
// fetched by LDS transpose reads, again shared by both row blocks.
// Workgroup ids are mapped so that each XCD owns a contiguous run of (kv head, split)
// streams: concurrently resident query tiles sweep the same prompt K/V tiles, which are
// then fetched from HBM once per XCD and served to its CUs from L2.
//
// replay_fwd_merge: log-sum-exp merge of the split partials,
//   lse = log sum_s exp(lse_s),  O = sum_s exp(lse_s - lse) O_s.
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

// Query rows per wave: 32 * RB. RB = 1 keeps two waves per SIMD resident (latency of one wave's
// softmax and LDS reads hidden behind the other's MFMAs); RB = 2 shares each LDS fragment between
// two MFMAs but leaves one wave per SIMD.
constexpr int kFwdRowBlocks = 1;

template <int D, int DV>
struct FwdCfg {
  static constexpr int RB = kFwdRowBlocks;
  static constexpr int BM = 128 * RB;         // packed query rows per workgroup
  static constexpr int BN = 64;               // keys per tile
  static constexpr int KCH = D / 8;           // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;
  static constexpr int KROW = D * 2;          // bytes per K row in LDS
  static constexpr int VROW = DV * 2;
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = BN * VROW;
  static constexpr int KINS = KBYTES / 1024 / 4;  // 1 KB direct-load instructions per wave per K tile
  static constexpr int VINS = VBYTES / 1024 / 4;
  static constexpr int KS = D / 16;           // MFMA k-steps over the head dim
  static constexpr int NB = DV / 32;          // 32-wide blocks of the value dim
};

template <int D, int DV>
__global__ __launch_bounds__(256, kFwdRowBlocks == 1 ? 2 : 1) void replay_fwd(FwdArgs a) {
  using C = FwdCfg<D, DV>;
  // two pipeline stages (64 KB at D = 128, so two workgroups fit in a CU's LDS)
  __shared__ __attribute__((aligned(1024))) char sK0[C::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[C::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[C::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[C::VBYTES];

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

  // two 32-row blocks per wave; one query row per lane in each
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
      // with one wave per SIMD, Q fragments (only ever MFMA operands) live in AGPRs, leaving
      // VGPRs for the accumulators and prefetched LDS fragments; at two waves per SIMD the
      // register file is split evenly and they stay in VGPRs
      if constexpr (C::RB == 2) asm volatile("" : "+a"(qf[rb][ks]));
    }
  }

  // lane-constant LDS byte offsets (the tile base and the 32-key block offset are added as immediates)
  int koff[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koff[ks] = l32 * C::KROW + (((2 * ks + hl) ^ swz<C::KCH>(l32)) << 4);
  int voff[2][C::NB];
  {
    const int jj = lane & 15;
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int row = 4 * hl + (jj >> 2) + 8 * sec;  // row within the 16-row group (mod 16)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int chunk = nb * 4 + 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
        voff[sec][nb] = row * C::VROW + ((chunk ^ swz<C::VCH>(row)) << 4) + (jj & 1) * 8;
      }
    }
  }

  // key range: prompt tiles of this split, then (last split) the response's causal tiles
  const int pt0 = sp * a.ptiles_per_split;
  const int np = max(0, min(a.ptiles, pt0 + a.ptiles_per_split) - pt0);
  const int t_lo = m0 / g;
  const int t_hi = (min(M, m0 + C::BM) - 1) / g;
  const int ns = (sp == a.splits - 1) ? (t_hi / C::BN + 1) : 0;
  const int nit = np + ns;

  auto tile_info = [&](int it, const uint16_t*& kb, const uint16_t*& vb, int& key0, int& nvalid, bool& sfx) {
    if (it < np) {
      key0 = (pt0 + it) * C::BN;
      nvalid = min(C::BN, G.P - key0);
      kb = G.Kp + (int64_t)key0 * G.ldk + kvh * D;
      vb = G.Vp + (int64_t)key0 * G.ldv + kvh * DV;
      sfx = false;
    } else {
      key0 = (it - np) * C::BN;
      nvalid = min(C::BN, R - key0);
      kb = G.Ks + (int64_t)(tokb + key0) * G.ldk + kvh * D;
      vb = G.Vs + (int64_t)(tokb + key0) * G.ldv + kvh * DV;
      sfx = true;
    }
  };
  // global -> LDS: each 1 KB instruction fills 1024 / (row bytes) consecutive rows; rows past the
  // valid keys re-read the last valid row (finite data, masked out of the softmax)
  auto issue_tile = [&](int it, char* kdst, char* vdst) {
    const uint16_t *kb, *vb;
    int key0, nvalid;
    bool sfx;
    tile_info(it, kb, vb, key0, nvalid, sfx);
#pragma unroll
    for (int u = 0; u < C::KINS; ++u) {
      const int ins = wv * C::KINS + u;
      const int row = ins * (64 / C::KCH) + lane / C::KCH;
      const int c = (lane % C::KCH) ^ swz<C::KCH>(row);
      lds_dma16(kb + (int64_t)min(row, nvalid - 1) * G.ldk + c * 8, kdst + ins * 1024);
    }
#pragma unroll
    for (int u = 0; u < C::VINS; ++u) {
      const int ins = wv * C::VINS + u;
      const int row = ins * (64 / C::VCH) + lane / C::VCH;
      const int c = (lane % C::VCH) ^ swz<C::VCH>(row);
      lds_dma16(vb + (int64_t)min(row, nvalid - 1) * G.ldv + c * 8, vdst + ins * 1024);
    }
  };

  f32x16 o[C::RB][C::NB];
  float m_run[C::RB], l_run[C::RB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) o[rb][nb] = f32x16{};
  }
  const float c2 = G.scale_log2;

  // only ragged prompt tiles and the response's diagonal tiles take the (wave-uniform) mask branch
  auto compute = [&](int it, const char* kbuf, const char* vbuf) {
    const uint16_t *kbp, *vbp;
    int key0, nvalid;
    bool sfx;
    tile_info(it, kbp, vbp, key0, nvalid, sfx);
    const bool causal = sfx && (key0 + C::BN - 1 > t_lo);
    const bool masked = causal || nvalid < C::BN;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st[C::RB];
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) st[rb] = f32x16{};
      bf16x8 vf[2][C::NB];
      if constexpr (C::RB == 2) {
        // one wave per SIMD: issue all K fragments of this 32-key block at once, then the
        // S^T = K Q^T MFMAs, then all V^T fragments (transposed LDS reads) so they are in flight
        // while the softmax runs
        bf16x8 kf[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) kf[ks] = lds_b128_at(kbuf, kb * 32 * C::KROW + koff[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
          for (int rb = 0; rb < C::RB; ++rb) st[rb] = mfma32(kf[ks], qf[rb][ks], st[rb]);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const int rowbase = (kb * 32 + 16 * hs) * C::VROW;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb)
            vf[hs][nb] = join_tr(lds_tr_at(vbuf, rowbase + voff[0][nb]), lds_tr_at(vbuf, rowbase + voff[1][nb]));
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // two waves per SIMD hide each other's latencies: plain per-fragment order
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) st[0] = mfma32(lds_b128_at(kbuf, kb * 32 * C::KROW + koff[ks]), qf[0][ks], st[0]);
      }
      if (masked) {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const bool bad = key >= nvalid || (causal && key0 + key > trow[rb]);
            st[rb][r] = bad ? -INFINITY : st[rb][r];
          }
      }
      // stage 4: online softmax, one row per lane (the other half-wave holds the row's other keys)
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[rb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run[rb], mx);
        const float ms = (m_new == -INFINITY ? 0.0f : m_new) * c2;
        const float alpha = fast_exp2(m_run[rb] * c2 - ms);
        m_run[rb] = m_new;
        if (__any(alpha != 1.0f)) {
          l_run[rb] *= alpha;
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) o[rb][nb] *= alpha;
        }
        float ls = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(st[rb][r], c2, -ms));
          st[rb][r] = p;
          ls += p;
        }
        l_run[rb] += ls;
      }
      // stage 5: O^T += V^T P^T; each V^T fragment feeds two MFMAs
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        bf16x8 pb[C::RB];
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) pb[rb] = c_regs_to_bf16x8(st[rb], 8 * hs);
        const int rowbase = (kb * 32 + 16 * hs) * C::VROW;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const bf16x8 va = C::RB == 2 ? vf[hs][nb]
                                       : join_tr(lds_tr_at(vbuf, rowbase + voff[0][nb]), lds_tr_at(vbuf, rowbase + voff[1][nb]));
#pragma unroll
          for (int rb = 0; rb < C::RB; ++rb) o[rb][nb] = mfma32(va, pb[rb], o[rb][nb]);
        }
      }
    }
  };

  // tile it+1 streams into the other stage while tile it is computed; the barrier after the
  // wait makes every wave's part of tile it visible and retires all reads of the stage refilled next
  if (nit > 0) issue_tile(0, sK0, sV0);
  for (int it = 0; it < nit; it += 2) {
    wait_vmem();
    __syncthreads();
    if (it + 1 < nit) issue_tile(it + 1, sK1, sV1);
    compute(it, sK0, sV0);
    if (it + 1 >= nit) break;
    wait_vmem();
    __syncthreads();
    if (it + 2 < nit) issue_tile(it + 2, sK0, sV0);
    compute(it + 1, sK1, sV1);
  }

#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const float l = l_run[rb] + __shfl_xor(l_run[rb], 32, 64);
    if (!rvalid[rb]) continue;
    const int64_t tok = tokb + trow[rb];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float lse = l > 0.0f ? m_run[rb] * G.scale + fast_log2(l) * kLn2 : -INFINITY;
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
