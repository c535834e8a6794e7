// Replay attention backward on gfx950 (LongStraw study notes §2-1 step 4, §2-2, §3-2 (4)): with
// P = exp(S scale - LSE), dP = dO V^T, Delta = rowsum(dO * O) and dS = P (dP - Delta),
//   dV_j += sum_rows P_rj dO_r,  dK_j += scale sum_rows dS_rj Q_r,  dQ_r = scale sum_j dS_rj K_j.
//
// Delta is taken from O + O_lo when the forward's rounding residual O_lo is given (O alone otherwise).
// This file holds the Delta pass (replay_bwd_pre) and the launch sequence of one backward call:
// Delta, then the dK/dV kernels (replay_attn_dkdv.hip: key-tile owners, prompt keys accumulated in
// place), then dQ (replay_attn_dq.hip: query-tile owners, split-K over the prompt).
#include "common.h"
#include "kernels.h"

namespace lsr {

namespace {

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
    u32x4 z = {0u, 0u, 0u, 0u};
    if (a.O_lo) z = *reinterpret_cast<const u32x4*>(a.O_lo + pair * DV + c * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s += bf16_lo(x[q]) * (bf16_lo(y[q]) + bf16_lo(z[q])) + bf16_hi(x[q]) * (bf16_hi(y[q]) + bf16_hi(z[q]));
  }
#pragma unroll
  for (int o = TPP / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (ok && c == 0) {
    const int64_t t = pair / G.Hq;
    const int h = (int)(pair % G.Hq);
    a.delta[(int64_t)h * G.T + t] = s;
  }
}

template <int D, int DV>
hipError_t bwd_go(BwdArgs& a, hipStream_t st) {
  const AttnGeom& G = a.geo;
  const long long threads = (long long)G.T * G.Hq * (DV / 8);
  hipLaunchKernelGGL((replay_bwd_pre<DV>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_bwd_dkdv(a, D, DV, st)) != hipSuccess) return e;
  return launch_bwd_dq(a, D, DV, st);
}

}  // namespace

hipError_t launch_attn_bwd(BwdArgs& a, int Dqk, int Dv, hipStream_t st) {
  if (Dqk == kWideDqk && Dv == kWideDv) return bwd_go<kWideDqk, kWideDv>(a, st);
  if (Dqk == 64 && Dv == 64) return bwd_go<64, 64>(a, st);
  if (Dqk == 128 && Dv == 128) return bwd_go<128, 128>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace lsr
