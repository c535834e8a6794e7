// Per-row scalar part of the clipped-GRPO token objective (LongStraw study notes, §1-1, L_policy
// equation), shared by the loss kernels over logits rows (grpo_loss.hip) and the LM-head kernels
// (lmhead.hip): everything that depends on a row's target logit and log-sum-exp only.
#pragma once
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace lsr {

// group advantage A and weight w = 1 / (G R_i) of the response holding launch-relative row `row`
__device__ __forceinline__ void row_coefs(const GrpoArgs& a, int64_t row, float* A, float* w) {
  int i = 0;
  while (i + 1 < a.n && row >= a.row_end[i]) ++i;
  *A = a.A[i];
  *w = a.w[i];
}

// logp = x_y - lse, rho = exp(logp - old), the clipped term and its flag; old_lp is the row's
// old_logp entry, which callers load at the start of the row so that its latency is hidden. The
// thread with `writer` set stores the row's loss term, log-prob and clip flag. Returns the dlogits
// coefficient c = clipped ? 0 : w A rho. A target outside [0, V) or NaN data make the row NaN.
__device__ __forceinline__ float row_scalar(const GrpoArgs& a, int64_t row, float xy, bool y_ok, float lse,
                                            float old_lp, bool writer) {
  float A, w;
  row_coefs(a, row, &A, &w);
  const float logp = y_ok ? xy - lse : __builtin_nanf("");
  const float rho = expf(logp - old_lp);
  const bool nan = !(rho == rho);
  const float unclipped = rho * A;
  const float clipped_v = fminf(fmaxf(rho, 1.0f - a.eps), 1.0f + a.eps) * A;
  const bool clipped = !nan && (clipped_v < unclipped);
  const float term = nan ? rho : fminf(unclipped, clipped_v);
  if (writer) {
    a.row_loss[row] = -w * term;
    if (a.logp_out) a.logp_out[row] = logp;
    if (a.clipped_out) a.clipped_out[row] = clipped ? 1 : 0;
  }
  return clipped ? 0.0f : w * A * rho;
}

}  // namespace lsr
