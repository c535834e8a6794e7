// ls_grpo_token_loss_noalloc: the clipped-GRPO token objective (LongStraw study notes, §1-1, L_policy
// equation) for callers that cannot allocate device memory. The objective's only scratch memory is
// one fp32 loss term per row, which the fixed-order reduction sums; here it lives in a file-scope
// device array instead of a caller workspace. The kernels, their launches and every result are
// those of ls_grpo_token_loss.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ls_replay.h"

namespace {

// One array per GPU the library runs on (each device holds its own copy of a __device__ variable),
// kept until the process ends. Calls on one GPU share it: each row's term is written before the
// reduction reads it, so nothing has to start at zero, and calls that overlap on one GPU race.
static __device__ __align__(256) float scratch[LS_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's array, looked up once per device with that device current. The
// array's name in host code is only a host-side stand-in: kernels get this address, never the name.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LS_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LS_OK;
}

}  // namespace

extern "C" int ls_grpo_token_loss_noalloc(void* stream, int32_t V, int32_t G, const int32_t* R, const float* rewards,
                                          float eps, int32_t first, int32_t count, const void* logits,
                                          const int32_t* targets, const float* old_logp, void* dlogits,
                                          float* loss_accum, float* logp_out, uint8_t* clipped_out) {
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != LS_OK) return st;
  // Same validation and launches as the workspace entry point; more rows than the array holds fail
  // its workspace-size check with LS_ERR_WORKSPACE before anything is launched.
  return ls_grpo_token_loss(stream, V, G, R, rewards, eps, first, count, logits, targets, old_logp, dlogits,
                            loss_accum, logp_out, clipped_out, ws, sizeof(float) * (size_t)LS_NOALLOC_MAX_ROWS);
}
