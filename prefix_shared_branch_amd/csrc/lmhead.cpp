// LM head fused with the clipped-GRPO token loss (host side): the step to the left of the loss. The
// objective (LongStraw study notes §1-1, L_policy) reads each token's logits row over the whole
// vocabulary; here the rows are formed from the hidden states, logits = H W^T, one chunk of tokens
// at a time, so the [T, V] logits of a response never exist at once:
//
//   for each chunk of kLmChunk tokens:
//     logits_c  = H_c W^T                (bf16 out, fp32 accumulation: a library GEMM)
//     dlogits_c = the fused loss kernel on logits_c (grpo_loss.hip; loss share, log-probs, clip flags)
//     dH_c      = dlogits_c W            (bf16 out)
//     dW       += dlogits_c^T H_c        (fp32 accumulator, added in place across chunks and calls)
//
// The three products are plain dense GEMMs and go to rocBLAS (gemm_ex, bf16 in, fp32 compute,
// atomics disabled so results are run-to-run identical); the logits and dlogits of one chunk live
// in the caller's workspace.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/ls_replay.h"
#include "kernels.h"

namespace {

constexpr int64_t kLmChunk = 2048;        // tokens per chunk
constexpr int32_t kLmMaxVocab = 1 << 24;  // the loss kernel's row limit
constexpr int kMaxDevices = 64;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct LmLayout {
  size_t logits, dlogits, row_loss, total;
};
LmLayout lm_layout(int64_t T, int32_t V) {
  const int64_t tc = T < kLmChunk ? T : kLmChunk;
  LmLayout l;
  l.logits = 0;
  l.dlogits = align256((size_t)tc * V * 2);
  l.row_loss = l.dlogits + align256((size_t)tc * V * 2);
  l.total = l.row_loss + align256(lsr::grpo_workspace_bytes(tc));
  return l;
}

// one rocBLAS handle per device, created on first use and kept for the process
std::mutex g_mu;
rocblas_handle g_handle[kMaxDevices] = {};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int ls_grpo_lmhead_workspace_bytes(int64_t T, int32_t V, int32_t d, size_t* bytes) {
  if (!bytes || T < 0 || V < 1 || d < 1) return LS_ERR_INVALID_ARG;
  *bytes = lm_layout(T, V).total;
  return LS_OK;
}

int ls_grpo_lmhead_loss(void* stream, int32_t V, int32_t d, int32_t G, const int32_t* R, const float* rewards,
                        float eps, int32_t first, int32_t count, const void* H, const void* W,
                        const int32_t* targets, const float* old_logp, float* loss_accum, void* dH,
                        float* dW_accum, float* logp_out, uint8_t* clipped_out, void* workspace,
                        size_t workspace_bytes) {
  if (V < 1 || d < 1 || G < 1 || !R || !rewards) return LS_ERR_INVALID_ARG;
  if (V > kLmMaxVocab) return LS_ERR_UNSUPPORTED;
  if ((V % 8) != 0 || (d % 8) != 0) return LS_ERR_UNSUPPORTED;   // 16-byte rows for the loss kernel
  if (!std::isfinite(eps) || !(eps > 0.0f) || !(eps < 1.0f)) return LS_ERR_INVALID_ARG;
  if (first < 0 || count < 1 || (int64_t)first + count > G) return LS_ERR_INVALID_ARG;
  for (int i = 0; i < G; ++i)
    if (R[i] < 1 || !std::isfinite(rewards[i])) return LS_ERR_INVALID_ARG;
  if ((dH == nullptr) != (dW_accum == nullptr)) return LS_ERR_INVALID_ARG;
  int64_t T = 0;
  for (int i = first; i < first + count; ++i) T += R[i];
  if (T > INT32_MAX || (int64_t)V * d > INT32_MAX) return LS_ERR_UNSUPPORTED;
  if (!H || !W || !targets || !old_logp || !loss_accum) return LS_ERR_INVALID_ARG;
  const void* a16[] = {H, W, dH, dW_accum};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return LS_ERR_INVALID_ARG;
  if (!aligned(targets, 4) || !aligned(old_logp, 4) || !aligned(loss_accum, 4) || (logp_out && !aligned(logp_out, 4)))
    return LS_ERR_INVALID_ARG;
  const LmLayout lay = lm_layout(T, V);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < lay.total) return LS_ERR_WORKSPACE;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LS_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_mu);   // the handle's stream is set per call
  rocblas_handle& h = g_handle[dev];
  if (!h) {
    if (rocblas_create_handle(&h) != rocblas_status_success) {
      h = nullptr;
      return LS_ERR_HIP;
    }
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) return LS_ERR_HIP;
  }
  if (rocblas_set_stream(h, st) != rocblas_status_success) return LS_ERR_HIP;

  char* ws = static_cast<char*>(workspace);
  uint16_t* logits = reinterpret_cast<uint16_t*>(ws + lay.logits);
  uint16_t* dlogits = reinterpret_cast<uint16_t*>(ws + lay.dlogits);
  float* row_loss = reinterpret_cast<float*>(ws + lay.row_loss);
  const uint16_t* Hb = static_cast<const uint16_t*>(H);
  uint16_t* dHb = static_cast<uint16_t*>(dH);
  const float one = 1.0f, zero = 0.0f;
  const bool grad = dH != nullptr;
  // rocBLAS is column-major: a row-major [r, c] array with row stride c is its [c, r] matrix
  for (int64_t c0 = 0; c0 < T; c0 += kLmChunk) {
    const int tc = (int)((T - c0) < kLmChunk ? (T - c0) : kLmChunk);
    // logits [tc, V] = H_c W^T  <=>  (V x tc) = op(W: d x V)^T (d x tc)
    if (rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, V, tc, d, &one, W,
                        rocblas_datatype_bf16_r, d, Hb + c0 * d, rocblas_datatype_bf16_r, d, &zero, logits,
                        rocblas_datatype_bf16_r, V, logits, rocblas_datatype_bf16_r, V, rocblas_datatype_f32_r,
                        rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
      return LS_ERR_HIP;
    const int rc = lsr::grpo_rows(st, V, G, R, rewards, eps, first, count, c0, c0 + tc, logits, targets, old_logp,
                                  grad ? dlogits : nullptr, loss_accum, logp_out, clipped_out, row_loss, true);
    if (rc != LS_OK) return rc;
    if (!grad) continue;
    // dH_c [tc, d] = dlogits_c W  <=>  (d x tc) = (d x V)(V x tc)
    if (rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, d, tc, V, &one, W,
                        rocblas_datatype_bf16_r, d, dlogits, rocblas_datatype_bf16_r, V, &zero, dHb + c0 * d,
                        rocblas_datatype_bf16_r, d, dHb + c0 * d, rocblas_datatype_bf16_r, d, rocblas_datatype_f32_r,
                        rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
      return LS_ERR_HIP;
    // dW [V, d] += dlogits_c^T H_c  <=>  (d x V) += (d x tc) op(dlogits: V x tc)^T
    if (rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_transpose, d, V, tc, &one, Hb + c0 * d,
                        rocblas_datatype_bf16_r, d, dlogits, rocblas_datatype_bf16_r, V, &one, dW_accum,
                        rocblas_datatype_f32_r, d, dW_accum, rocblas_datatype_f32_r, d, rocblas_datatype_f32_r,
                        rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
      return LS_ERR_HIP;
  }
  return LS_OK;
}

}  // extern "C"
