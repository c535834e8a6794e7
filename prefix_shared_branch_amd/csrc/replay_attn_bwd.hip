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
// dQ (query-tile owner, split-K over the prompt) is in replay_attn_dq.hip.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

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
  return launch_bwd_dq(a, D, DV, st);
}

}  // namespace

hipError_t launch_attn_bwd(BwdArgs& a, int Dqk, int Dv, hipStream_t st) {
  if (Dqk == 64 && Dv == 64) return bwd_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return bwd_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
