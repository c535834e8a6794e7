// Replay attention backward on gfx950. The prompt-side gradient is the d l / d z_P term of
// the gradient decomposition in the LongStraw study notes (§2-2); serial replay adds it
// into resident accumulators response after response (§2-1 step 4, §3-2 (4)), and the
// accumulators are owned by the prompt pages they belong to (§4-3 (2), page-owner dK/dV).
//
// With P = exp(S*scale - LSE), dP = dO V^T, Delta = rowsum(dO * O), dS = P (dP - Delta):
//   dV_j += sum_rows P_rj dO_r,  dK_j += scale sum_rows dS_rj Q_r,  dQ_r = scale sum_j dS_rj K_j.
//
// replay_bwd_pre   Delta per (token, head).
// replay_bwd_dkdv  key-tile owner: one workgroup = 4 waves x 32 keys of one kv head, holding
//                  K, V fragments and the dK, dV accumulators in registers while it sweeps all
//                  query rows that see those keys (32 rows per step, staged through LDS).
//                  Prompt tiles: fp32 read-modify-write into dKp/dVp (each element written by
//                  exactly one workgroup per call); P and dS enter the MFMAs as a bf16 hi/lo
//                  pair so the fp32 accumulators keep ~16 significant bits per term.
//                  Suffix tiles: causal, bf16 dKs/dVs stores.
// replay_bwd_dq    query-tile owner with split-K over the prompt (like the forward);
//                  recomputes S and dP per key tile; partials summed in fixed order.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

// hi = bf16(x), lo = bf16(x - hi) for 8 consecutive C registers
__device__ __forceinline__ void split_bf16x8(const f32x16& c, int r0, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = (__bf16)c[r0 + j];
    hi[j] = h;
    lo[j] = (__bf16)(c[r0 + j] - (float)h);
  }
}

// ------------------------------------------------------------------ Delta = rowsum(dO * O)
template <int DV>
__global__ __launch_bounds__(256) void replay_bwd_pre(BwdArgs a) {
  constexpr int TPP = DV / 8;  // threads per (token, head)
  const AttnGeom& G = a.geo;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pair = idx / TPP;
  const int c = (int)(idx % TPP);
  const bool ok = pair < (int64_t)G.T * G.Hq;
  float s = 0.0f;
  if (ok) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(a.dO + pair * DV + c * 8);
    const u32x4 y = *reinterpret_cast<const u32x4*>(a.O + pair * DV + c * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) s += bf16_lo(x[q]) * bf16_lo(y[q]) + bf16_hi(x[q]) * bf16_hi(y[q]);
  }
#pragma unroll
  for (int o = TPP / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (ok && c == 0) {
    const int64_t t = pair / G.Hq;
    const int h = (int)(pair % G.Hq);
    a.delta[(int64_t)h * G.T + t] = s;
  }
}

// ------------------------------------------------------------------ dK / dV (key owner)
template <int D, int DV>
struct DkvCfg {
  static constexpr int BN = 128;       // keys per workgroup (32 per wave)
  static constexpr int BR = 32;        // query rows per step
  static constexpr int NT = 256;
  static constexpr int QP = D + 8;     // LDS pitches
  static constexpr int OP = DV + 8;
  static constexpr int KS = D / 16;
  static constexpr int VS = DV / 16;
  static constexpr int DB = D / 32;
  static constexpr int VB = DV / 32;
  static constexpr int QCH = BR * D / 8 / NT;
  static constexpr int OCH = BR * DV / 8 / NT;
};

template <int D, int DV, bool PROMPT>
__global__ __launch_bounds__(256, 1) void replay_bwd_dkdv(BwdArgs a) {
  using C = DkvCfg<D, DV>;
  static_assert(C::QCH >= 1 && C::OCH >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][C::BR * C::QP];
  __shared__ __attribute__((aligned(16))) uint16_t sO[2][C::BR * C::OP];
  __shared__ __attribute__((aligned(16))) float sL[2][C::BR];
  __shared__ __attribute__((aligned(16))) float sD[2][C::BR];

  const AttnGeom& G = a.geo;
  const int nk = PROMPT ? a.ktiles_prompt : a.ktile0[G.n_resp];
  const int W = nk * G.Hkv;
  const int per_xcd = (W + 7) >> 3;
  const int w = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (w >= W) return;
  const int kvh = w / nk;
  const int kt = w - kvh * nk;
  const int g = G.g;

  int key0, nkeys, tokb = 0, R = 0, row_begin, row_end;
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
    key0 = (kt - a.ktile0[ri]) * C::BN;  // within the response
    nkeys = min(C::BN, R - key0);
    row_begin = (tokb + key0) * g;
    row_end = (tokb + R) * g;
  }

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int hl = lane >> 5;
  const int mykey = wv * 32 + (lane & 31);  // within the tile
  const bool kvalid = mykey < nkeys;

  // K, V fragments of this wave's 32 keys (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[C::KS], vf[C::VS];
  {
    const uint16_t* kr = PROMPT ? G.Kp + (int64_t)(key0 + mykey) * G.ldk + kvh * D
                                : G.Ks + (int64_t)(tokb + key0 + mykey) * G.ldk + kvh * D;
    const uint16_t* vr = PROMPT ? G.Vp + (int64_t)(key0 + mykey) * G.ldv + kvh * DV
                                : G.Vs + (int64_t)(tokb + key0 + mykey) * G.ldv + kvh * DV;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kf[ks] = kvalid ? ld_bf16x8(kr + ks * 16 + hl * 8) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) vf[ks] = kvalid ? ld_bf16x8(vr + ks * 16 + hl * 8) : zero_bf16x8();
  }

  f32x16 dk[C::DB], dv[C::VB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b) dk[b] = f32x16{};
#pragma unroll
  for (int b = 0; b < C::VB; ++b) dv[b] = f32x16{};

  u32x4 qreg[C::QCH], oreg[C::OCH];
  float lreg = 0.0f, dreg = 0.0f;
  auto load_rows = [&](int rb) {
#pragma unroll
    for (int u = 0; u < C::QCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      const int i = c / (D / 8), col = c % (D / 8);
      const int m = rb + i;
      if (m < row_end) {
        const int tg = m / g, h = kvh * g + (m - tg * g);
        qreg[u] = *reinterpret_cast<const u32x4*>(G.Q + ((int64_t)tg * G.Hq + h) * D + col * 8);
      } else {
        qreg[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < C::OCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      const int i = c / (DV / 8), col = c % (DV / 8);
      const int m = rb + i;
      if (m < row_end) {
        const int tg = m / g, h = kvh * g + (m - tg * g);
        oreg[u] = *reinterpret_cast<const u32x4*>(a.dO + ((int64_t)tg * G.Hq + h) * DV + col * 8);
      } else {
        oreg[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (threadIdx.x < C::BR) {
      const int m = rb + threadIdx.x;
      if (m < row_end) {
        const int tg = m / g, h = kvh * g + (m - tg * g);
        lreg = a.lse[(int64_t)h * G.T + tg] * kLog2e;
        dreg = a.delta[(int64_t)h * G.T + tg];
      } else {
        lreg = INFINITY;  // P = 0 for padding rows
        dreg = 0.0f;
      }
    }
  };
  auto store_rows = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::QCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      *reinterpret_cast<u32x4*>(&sQ[buf][(c / (D / 8)) * C::QP + (c % (D / 8)) * 8]) = qreg[u];
    }
#pragma unroll
    for (int u = 0; u < C::OCH; ++u) {
      const int c = threadIdx.x + u * C::NT;
      *reinterpret_cast<u32x4*>(&sO[buf][(c / (DV / 8)) * C::OP + (c % (DV / 8)) * 8]) = oreg[u];
    }
    if (threadIdx.x < C::BR) {
      sL[buf][threadIdx.x] = lreg;
      sD[buf][threadIdx.x] = dreg;
    }
  };

  const float c2 = G.scale_log2;
  const int nsteps = row_end > row_begin ? (row_end - row_begin + C::BR - 1) / C::BR : 0;
  if (nsteps > 0) {
    load_rows(row_begin);
    store_rows(0);
  }
  __syncthreads();
  const int jj = lane & 15;
  const int n0l = 16 * ((lane >> 4) & 1) + 4 * (jj & 3);
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const int rb = row_begin + step * C::BR;
    if (step + 1 < nsteps) load_rows(rb + C::BR);

    // S[row][key] and dP[row][key]: lane holds key (lane & 31), rows 8(r/4) + 4hl + r%4
    f32x16 s = f32x16{}, dp = f32x16{};
    const uint16_t* qa = &sQ[buf][(lane & 31) * C::QP + hl * 8];
    const uint16_t* oa = &sO[buf][(lane & 31) * C::OP + hl * 8];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) s = mfma32(lds_read_b128(qa + ks * 16), kf[ks], s);
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) dp = mfma32(lds_read_b128(oa + ks * 16), vf[ks], dp);

    f32x16 p, ds;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[buf][8 * q + 4 * hl]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[buf][8 * q + 4 * hl]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q + e;
        float pv = fast_exp2(__builtin_fmaf(s[r], c2, -l4[e]));
        bool vis = kvalid;
        if (!PROMPT) {
          const int row = rb + 8 * q + 4 * hl + e;
          const int t = row / g - tokb;  // token within the response
          vis = vis && (key0 + mykey <= t);
        }
        pv = vis ? pv : 0.0f;
        p[r] = pv;
        ds[r] = pv * (dp[r] - d4[e]);
      }
    }

    // dV^T[dv][key] += dO^T P,  dK^T[d][key] += Q^T dS  (A operands by LDS transpose reads)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int k0 = 16 * hs + 4 * hl + (jj >> 2);
      const uint16_t* otr = &sO[buf][k0 * C::OP + n0l];
      const uint16_t* qtr = &sQ[buf][k0 * C::QP + n0l];
      if (PROMPT) {
        bf16x8 ph, pl, dh, dl;
        split_bf16x8(p, 8 * hs, ph, pl);
        split_bf16x8(ds, 8 * hs, dh, dl);
#pragma unroll
        for (int b = 0; b < C::VB; ++b) {
          const bf16x8 at = join_tr(lds_read_tr(otr + b * 32), lds_read_tr(otr + b * 32 + 8 * C::OP));
          dv[b] = mfma32(at, ph, dv[b]);
          dv[b] = mfma32(at, pl, dv[b]);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
          const bf16x8 at = join_tr(lds_read_tr(qtr + b * 32), lds_read_tr(qtr + b * 32 + 8 * C::QP));
          dk[b] = mfma32(at, dh, dk[b]);
          dk[b] = mfma32(at, dl, dk[b]);
        }
      } else {
        const bf16x8 pb = c_regs_to_bf16x8(p, 8 * hs);
        const bf16x8 db = c_regs_to_bf16x8(ds, 8 * hs);
#pragma unroll
        for (int b = 0; b < C::VB; ++b) {
          const bf16x8 at = join_tr(lds_read_tr(otr + b * 32), lds_read_tr(otr + b * 32 + 8 * C::OP));
          dv[b] = mfma32(at, pb, dv[b]);
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
          const bf16x8 at = join_tr(lds_read_tr(qtr + b * 32), lds_read_tr(qtr + b * 32 + 8 * C::QP));
          dk[b] = mfma32(at, db, dk[b]);
        }
      }
    }
    if (step + 1 < nsteps) store_rows(buf ^ 1);
    __syncthreads();
  }

  if (!kvalid) return;
  // C layout of dV^T / dK^T: lane holds key (lane & 31), dims 32b + 8(r/4) + 4hl + r%4
  const float sc = G.scale;
  if (PROMPT) {
    float* dvr = a.dVp + ((int64_t)(key0 + mykey) * G.Hkv + kvh) * DV + 4 * hl;
    float* dkr = a.dKp + ((int64_t)(key0 + mykey) * G.Hkv + kvh) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::VB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dvr + b * 32 + 8 * q);
        const f32x4 add = {dv[b][4 * q], dv[b][4 * q + 1], dv[b][4 * q + 2], dv[b][4 * q + 3]};
        *ptr = *ptr + add;
      }
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4* ptr = reinterpret_cast<f32x4*>(dkr + b * 32 + 8 * q);
        const f32x4 add = {dk[b][4 * q] * sc, dk[b][4 * q + 1] * sc, dk[b][4 * q + 2] * sc, dk[b][4 * q + 3] * sc};
        *ptr = *ptr + add;
      }
  } else {
    const int64_t tok = tokb + key0 + mykey;
    uint16_t* dvr = a.dVs + (tok * G.Hkv + kvh) * DV + 4 * hl;
    uint16_t* dkr = a.dKs + (tok * G.Hkv + kvh) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::VB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v = {pack_bf16x2(dv[b][4 * q], dv[b][4 * q + 1]), pack_bf16x2(dv[b][4 * q + 2], dv[b][4 * q + 3])};
        *reinterpret_cast<u32x2*>(dvr + b * 32 + 8 * q) = v;
      }
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v = {pack_bf16x2(dk[b][4 * q] * sc, dk[b][4 * q + 1] * sc),
                         pack_bf16x2(dk[b][4 * q + 2] * sc, dk[b][4 * q + 3] * sc)};
        *reinterpret_cast<u32x2*>(dkr + b * 32 + 8 * q) = v;
      }
  }
}

// ------------------------------------------------------------------ dQ (query owner, split-K)
template <int D, int DV>
struct DqCfg {
  static constexpr int BM = 128;              // packed query rows per workgroup (32 per wave)
  static constexpr int BN = 64;               // keys per tile
  static constexpr int KCH = D / 8;           // 16-byte chunks per row
  static constexpr int VCH = DV / 8;
  static constexpr int KP = KCH + 1;          // padded pitches in chunks (row-wise reads conflict-free)
  static constexpr int VP = VCH + 1;
  static constexpr int KROW = KP * 16;        // LDS bytes per row
  static constexpr int VROW = VP * 16;
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = BN * VROW;
  static constexpr int KS = D / 16;
  static constexpr int VS = DV / 16;
  static constexpr int DB = D / 32;
};

// Two workgroups per CU (68 KB of LDS each, <= 256 registers per wave) so that the two waves on a
// SIMD hide each other's LDS and softmax latency. K and V tiles stream global -> LDS by DMA into
// padded rows; K is read both row-wise (S^T = K Q^T) and transposed (dQ^T = K^T dS^T).
template <int D, int DV>
__global__ __launch_bounds__(256, 2) void replay_bwd_dq(BwdArgs a) {
  using C = DqCfg<D, DV>;
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
  const int mrow = m0 + wv * 32 + l32;
  const bool rvalid = mrow < M;
  const int trow = rvalid ? mrow / g : 0;
  const int hq = kvh * g + (rvalid ? mrow - trow * g : 0);
  const int64_t tok = tokb + trow;

  bf16x8 qf[C::KS], of[C::VS];
  {
    const uint16_t* qrow = G.Q + (tok * G.Hq + hq) * D + hl * 8;
    const uint16_t* orow = a.dO + (tok * G.Hq + hq) * DV + hl * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = rvalid ? ld_bf16x8(qrow + ks * 16) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < C::VS; ++ks) of[ks] = rvalid ? ld_bf16x8(orow + ks * 16) : zero_bf16x8();
  }
  const float lrow = rvalid ? a.lse[(int64_t)hq * G.T + tok] * kLog2e : INFINITY;
  const float drow = rvalid ? a.delta[(int64_t)hq * G.T + tok] : 0.0f;

  // lane-constant LDS byte offsets; row-wise reads of K and V share one table (same row length)
  // per-lane LDS bases; every fragment adds a compile-time immediate
  const int rbk = l32 * C::KROW + hl * 16;   // row-wise reads of K (key l32, 8 dims at 16ks + 8hl)
  const int rbv = l32 * C::VROW + hl * 16;   // row-wise reads of V
  // transposed reads of K: row 4hl + jj/4 (+ 8 sec + 16 hs + 32 kb), column 16 (lane/16 % 2) + 4 (jj % 4) (+ 32 b)
  const int tbk = (4 * hl + ((lane & 15) >> 2)) * C::KROW + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

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
  auto issue_tile = [&](int it, char* kdst, char* vdst) {
    const uint16_t *kb, *vb;
    int key0, nvalid;
    bool sfx;
    tile_info(it, kb, vb, key0, nvalid, sfx);
    dma_tile64<C::KCH, C::KP>(kb, G.ldk, nvalid, kdst, wv, lane);
    dma_tile64<C::VCH, C::VP>(vb, G.ldv, nvalid, vdst, wv, lane);
  };

  f32x16 dq[C::DB];
#pragma unroll
  for (int b = 0; b < C::DB; ++b) dq[b] = f32x16{};
  const float c2 = G.scale_log2;

  // MASK is a compile-time flag: only ragged prompt tiles and the response's diagonal tiles take
  // the masked body; everywhere else the softmax has no per-element conditions at all
  auto compute_body = [&](auto mask_tag, const char* kbuf, const char* vbuf, int key0, int nvalid, bool causal) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // Fragments stream in groups of four: each group's LDS reads are in flight while the
      // previous group's MFMAs run, so at most two groups (32 registers) are live at once.
      // S^T[key][row] = K Q^T, dP^T = V dO^T: lane holds row (lane & 31), keys 8(r/4) + 4hl + r%4
      constexpr int NG = C::KS / 2;  // fragments per group; equals the number of 32-wide dQ blocks
      static_assert(C::KS == C::VS && NG == C::DB, "grouping assumes Dqk == Dv");
      const char* kr = kbuf + kb * 32 * C::KROW;
      const char* vr = vbuf + kb * 32 * C::VROW;
      bf16x8 g0[NG], g1[NG];
#pragma unroll
      for (int i = 0; i < NG; ++i) g0[i] = lds_b128_at(kr + i * 32, rbk);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NG; ++i) g1[i] = lds_b128_at(kr + (NG + i) * 32, rbk);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int i = 0; i < NG; ++i) s = mfma32(g0[i], qf[i], s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NG; ++i) g0[i] = lds_b128_at(vr + i * 32, rbv);
#pragma unroll
      for (int i = 0; i < NG; ++i) s = mfma32(g1[i], qf[NG + i], s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NG; ++i) g1[i] = lds_b128_at(vr + (NG + i) * 32, rbv);
#pragma unroll
      for (int i = 0; i < NG; ++i) dp = mfma32(g0[i], of[i], dp);
      __builtin_amdgcn_sched_barrier(0);
      // transposed K fragments (first half of the keys) in flight while dS is formed
      auto tr_frags = [&](int hs, bf16x8* tf) {
        const char* kt = kbuf + (kb * 32 + 16 * hs) * C::KROW;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
          tf[b] = join_tr(lds_tr_at(kt + b * 64, tbk), lds_tr_at(kt + 8 * C::KROW + b * 64, tbk));
      };
      tr_frags(0, g0);
#pragma unroll
      for (int i = 0; i < NG; ++i) dp = mfma32(g1[i], of[NG + i], dp);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        float pv = fast_exp2(__builtin_fmaf(s[r], c2, -lrow));
        if constexpr (MASK) pv = (key >= nvalid || (causal && key0 + key > trow)) ? 0.0f : pv;
        ds[r] = pv * (dp[r] - drow);
      }
      // dQ^T[d][row] += K^T dS^T (second half's fragments load under the first half's MFMAs)
      tr_frags(1, g1);
      {
        const bf16x8 db = c_regs_to_bf16x8(ds, 0);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) dq[b] = mfma32(g0[b], db, dq[b]);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        const bf16x8 db = c_regs_to_bf16x8(ds, 8);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) dq[b] = mfma32(g1[b], db, dq[b]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto compute = [&](int it, const char* kbuf, const char* vbuf) {
    const uint16_t *kbp, *vbp;
    int key0, nvalid;
    bool sfx;
    tile_info(it, kbp, vbp, key0, nvalid, sfx);
    const bool causal = sfx && (key0 + C::BN - 1 > t_lo);
    if (causal || nvalid < C::BN) compute_body(std::true_type{}, kbuf, vbuf, key0, nvalid, causal);
    else compute_body(std::false_type{}, kbuf, vbuf, key0, nvalid, causal);
  };

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

  if (!rvalid) return;
  // C layout of dQ^T: lane holds row (lane & 31), dims 32b + 8(r/4) + 4hl + r%4
  const float sc = G.scale;
  if (a.splits == 1) {
    uint16_t* dst = a.dQ + (tok * G.Hq + hq) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 v = {pack_bf16x2(dq[b][4 * q] * sc, dq[b][4 * q + 1] * sc),
                         pack_bf16x2(dq[b][4 * q + 2] * sc, dq[b][4 * q + 3] * sc)};
        *reinterpret_cast<u32x2*>(dst + b * 32 + 8 * q) = v;
      }
  } else {
    float* dst = a.dq_part + (((int64_t)sp * G.T + tok) * G.Hq + hq) * D + 4 * hl;
#pragma unroll
    for (int b = 0; b < C::DB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {dq[b][4 * q], dq[b][4 * q + 1], dq[b][4 * q + 2], dq[b][4 * q + 3]};
        *reinterpret_cast<f32x4*>(dst + b * 32 + 8 * q) = v;
      }
  }
}

template <int D>
__global__ __launch_bounds__(256) void replay_bwd_dq_reduce(BwdArgs a) {
  const AttnGeom& G = a.geo;
  const int64_t n4 = (int64_t)G.T * G.Hq * D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n4) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) acc += reinterpret_cast<const f32x4*>(a.dq_part)[(int64_t)s * n4 + idx];
  acc *= G.scale;
  const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  reinterpret_cast<u32x2*>(a.dQ)[idx] = v;
}

template <int D, int DV>
hipError_t bwd_go(BwdArgs& a, hipStream_t st) {
  const AttnGeom& G = a.geo;
  hipError_t e;
  {
    const long long threads = (long long)G.T * G.Hq * (DV / 8);
    hipLaunchKernelGGL((replay_bwd_pre<DV>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.ktiles_prompt > 0) {
    const long long W = (long long)a.ktiles_prompt * G.Hkv;
    timer_mark(LS_KERNEL_DKDV_PROMPT, st, false);
    hipLaunchKernelGGL((replay_bwd_dkdv<D, DV, true>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(256), 0, st, a);
    timer_mark(LS_KERNEL_DKDV_PROMPT, st, true);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    const long long W = (long long)a.ktile0[G.n_resp] * G.Hkv;
    if (W > 0) {
      hipLaunchKernelGGL((replay_bwd_dkdv<D, DV, false>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(256), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  {
    const long long W = (long long)a.qtiles * G.Hkv * a.splits;
    if (W > 0) {
      timer_mark(LS_KERNEL_DQ, st, false);
      hipLaunchKernelGGL((replay_bwd_dq<D, DV>), dim3((unsigned)(((W + 7) / 8) * 8)), dim3(256), 0, st, a);
      timer_mark(LS_KERNEL_DQ, st, true);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (a.splits > 1) {
    const long long n4 = (long long)G.T * G.Hq * D / 4;
    hipLaunchKernelGGL((replay_bwd_dq_reduce<D>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_bwd(BwdArgs& a, int Dqk, int Dv, hipStream_t st) {
  if (Dqk == 64 && Dv == 64) return bwd_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return bwd_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
