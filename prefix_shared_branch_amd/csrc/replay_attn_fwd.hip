// Replay attention forward on gfx950 (LongStraw study notes, §2-1 step 4 and §3-2 (2)/(4)):
// the queries of one response attend to all prompt keys and, causally, to the response's
// own keys.
//
// replay_fwd: one workgroup = 4 waves = 128 GQA-packed query rows of one kv head, over the
// prompt key tiles of one split (plus, in the last split, the response's causal key tiles).
// Per 64-key tile:  K, V tiles are staged global -> VGPR -> LDS (double-buffered, padded
// rows); each wave computes S^T = K Q^T (MFMA 32x32x16 bf16, Q fragments held in VGPRs,
// K read from LDS), an online softmax whose row statistics are lane-local (one query row
// per lane), and O^T += V^T P^T with V^T fetched by LDS transpose reads.
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

template <int D, int DV>
struct FwdCfg {
  static constexpr int BM = 128;         // packed query rows per workgroup
  static constexpr int BN = 64;          // keys per tile
  static constexpr int NT = 256;
  static constexpr int KP = D + 8;       // LDS row pitch (elements) of the K tile
  static constexpr int VPT = DV + 8;     // LDS row pitch of the V tile
  static constexpr int KS = D / 16;      // MFMA k-steps over the head dim
  static constexpr int NB = DV / 32;     // 32-wide blocks of the value dim
  static constexpr int KCH = BN * D / 8 / NT;
  static constexpr int VCH = BN * DV / 8 / NT;
};

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

template <int D, int DV>
__global__ __launch_bounds__(256, 2) void replay_fwd(FwdArgs a) {
  using C = FwdCfg<D, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][C::BN * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][C::BN * C::VPT];

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
  const int mrow = m0 + wv * 32 + (lane & 31);
  const bool rvalid = mrow < M;
  const int trow = rvalid ? mrow / g : 0;
  const int hq = kvh * g + (rvalid ? mrow - trow * g : 0);

  bf16x8 qf[C::KS];
  {
    const uint16_t* qrow = G.Q + ((int64_t)(tokb + trow) * G.Hq + hq) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (rvalid) qf[ks] = ld_bf16x8(qrow + ks * 16);
      else qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  // key range: prompt tiles of this split, then (last split) the response's causal tiles
  const int pt0 = sp * a.ptiles_per_split;
  const int np = max(0, min(a.ptiles, pt0 + a.ptiles_per_split) - pt0);
  const int t_lo = m0 / g;
  const int t_hi = (min(M, m0 + C::BM) - 1) / g;
  const int ns = (sp == a.splits - 1) ? (t_hi / C::BN + 1) : 0;
  const int nit = np + ns;

  u32x4 kreg[C::KCH], vreg[C::VCH];
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
  auto load_tile = [&](int it) {
    const uint16_t *kb, *vb;
    int key0, nvalid;
    bool sfx;
    tile_info(it, kb, vb, key0, nvalid, sfx);
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      const int row = c / (D / 8), col = c % (D / 8);
      kreg[u] = row < nvalid ? *reinterpret_cast<const u32x4*>(kb + (int64_t)row * G.ldk + col * 8)
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < C::VCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      const int row = c / (DV / 8), col = c % (DV / 8);
      vreg[u] = row < nvalid ? *reinterpret_cast<const u32x4*>(vb + (int64_t)row * G.ldv + col * 8)
                             : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::KCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      const int row = c / (D / 8), col = c % (D / 8);
      *reinterpret_cast<u32x4*>(&sK[buf][row * C::KP + col * 8]) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < C::VCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      const int row = c / (DV / 8), col = c % (DV / 8);
      *reinterpret_cast<u32x4*>(&sV[buf][row * C::VPT + col * 8]) = vreg[u];
    }
  };

  f32x16 o[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) o[nb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float c2 = G.scale_log2;

  if (nit > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int buf = it & 1;
    if (it + 1 < nit) load_tile(it + 1);
    const uint16_t *kbp, *vbp;
    int key0, nvalid;
    bool sfx;
    tile_info(it, kbp, vbp, key0, nvalid, sfx);
    const bool causal = sfx && (key0 + C::BN - 1 > t_lo);
    const bool need_mask = causal || nvalid < C::BN;

    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = f32x16{};
      const uint16_t* kr = &sK[buf][(kb * 32 + (lane & 31)) * C::KP + hl * 8];
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) st[kb] = mfma32(lds_read_b128(kr + ks * 16), qf[ks], st[kb]);
    }
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool bad = key >= nvalid || (causal && key0 + key > trow);
          if (bad) st[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float ms = (m_new == -INFINITY ? 0.0f : m_new) * c2;
    const float alpha = fast_exp2(m_run * c2 - ms);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) o[nb] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(st[kb][r], c2, -ms));
        st[kb][r] = p;
        l_run += p;
      }
    // O^T += V^T P^T
    const int jj = lane & 15;
    const int n0l = 16 * ((lane >> 4) & 1) + 4 * (jj & 3);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const bf16x8 pb = c_regs_to_bf16x8(st[kb], 8 * hs);
        const int k0 = kb * 32 + 16 * hs + 4 * hl + (jj >> 2);
        const uint16_t* vr = &sV[buf][k0 * C::VPT + n0l];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const s16x4 t0 = lds_read_tr(vr + nb * 32);
          const s16x4 t1 = lds_read_tr(vr + nb * 32 + 8 * C::VPT);
          o[nb] = mfma32(join_tr(t0, t1), pb, o[nb]);
        }
      }
    if (it + 1 < nit) store_tile(buf ^ 1);
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 32, 64);
  if (!rvalid) return;
  const int64_t tok = tokb + trow;
  const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  const float lse = l_run > 0.0f ? m_run * G.scale + fast_log2(l_run) * kLn2 : -INFINITY;
  if (a.splits == 1) {
    uint16_t* orow = a.O + (tok * G.Hq + hq) * DV + 4 * hl;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v = {pack_bf16x2(o[nb][4 * q] * inv, o[nb][4 * q + 1] * inv),
                         pack_bf16x2(o[nb][4 * q + 2] * inv, o[nb][4 * q + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + nb * 32 + 8 * q) = v;
      }
    if (hl == 0) a.lse[(int64_t)hq * G.T + tok] = lse;
  } else {
    float* orow = a.o_part + (((int64_t)sp * G.T + tok) * G.Hq + hq) * DV + 4 * hl;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {o[nb][4 * q] * inv, o[nb][4 * q + 1] * inv, o[nb][4 * q + 2] * inv,
                         o[nb][4 * q + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + nb * 32 + 8 * q) = v;
      }
    if (hl == 0) a.lse_part[((int64_t)sp * G.Hq + hq) * G.T + tok] = lse;
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
  hipLaunchKernelGGL((replay_fwd<D, DV>), dim3((unsigned)(per_xcd * 8)), dim3(256), 0, st, a);
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
