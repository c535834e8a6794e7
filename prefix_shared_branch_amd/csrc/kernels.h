// Internal launch interface between the host API (api.cpp) and the gfx950 kernels.
// Host code validates every argument before calling these; the launchers assume valid input.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ls_replay.h"

namespace lsr {

constexpr int kMaxResp = 64;

// ---------------------------------------------------------------- GRPO token loss
struct GrpoArgs {
  const uint16_t* logits;   // bf16 [T, V]
  const int32_t* targets;   // [T]
  const float* old_logp;    // [T]
  uint16_t* dlogits;        // bf16 [T, V]
  float* row_loss;          // workspace [T]: -w_i * term_t
  float* logp_out;          // [T] or null
  uint8_t* clipped_out;     // [T] or null
  float* loss_accum;        // scalar, += sum of row_loss
  int64_t T;
  int32_t V;
  float eps;
  int32_t n;                     // responses in this launch
  int32_t row_end[kMaxResp];     // exclusive end row of each response (launch-relative)
  float A[kMaxResp];             // group advantage of each response
  float w[kMaxResp];             // 1 / (G * R_i)
};
// vec: rows are 16-byte aligned and V % 8 == 0
hipError_t launch_grpo(const GrpoArgs& a, bool vec, hipStream_t st);
size_t grpo_workspace_bytes(int64_t T);

// ---------------------------------------------------------------- replay attention
// Query rows are GQA-packed per kv head: within response i, packed row m = t * g + j is
// token t, query head kvh * g + j (g = Hq / Hkv).
struct AttnGeom {
  const uint16_t* Kp;
  const uint16_t* Vp;
  const uint16_t* Q;
  const uint16_t* Ks;
  const uint16_t* Vs;
  int64_t ldk, ldv;
  int32_t P, Hq, Hkv, g, T;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  int32_t n_resp;
  int32_t tok0[kMaxResp + 1];   // cu_seqlens
};

// Dimension-major repacking of key-major K or V rows (pack.hip): see launch_pack_keys_t.
struct PackArgs {
  const uint16_t* src;   // [rows, ld] bf16; head h, dim d of row r at src[r * ld + h * dim + d]
  int64_t ld;
  int32_t dim, heads;    // dim a multiple of 64
  int32_t nseg;          // 1 .. kMaxResp segments
  int64_t row0[kMaxResp];  // first source row of each segment
  int32_t n[kMaxResp];     // keys of each segment
  int64_t col0[kMaxResp];  // first output slot of each segment (multiple of 64, increasing)
  uint16_t* out;         // [heads * dim, out_ld] bf16
  int64_t out_ld;        // slots per output row (multiple of 64)
  int64_t cols;          // slots written per row (= out_ld)
};
hipError_t launch_pack_keys_t(const PackArgs& a, hipStream_t st);

struct FwdArgs {
  AttnGeom geo;
  uint16_t* O;          // bf16 [T, Hq, Dv]
  float* lse;           // [Hq, T]
  float* o_part;        // [S, T, Hq, Dv] fp32 (S > 1)
  float* lse_part;      // [S, Hq, T] (S > 1)
  const uint16_t* VTp;  // packed prompt V: [Hkv * Dv, ppad] (pack.hip layout)
  const uint16_t* VTs;  // packed response V: [Hkv * Dv, tpad], response i from slot spos[i]
  int64_t ppad, tpad;
  int32_t spos[kMaxResp + 1];
  int32_t splits;       // S
  int32_t ptiles;       // prompt key tiles
  int32_t ptiles_per_split;
  int32_t qtiles;       // query tiles per kv head (all responses)
  int32_t tile0[kMaxResp + 1];  // first query tile of each response
};

struct BwdArgs {
  AttnGeom geo;
  const uint16_t* O;
  const float* lse;
  const uint16_t* dO;
  uint16_t* dQ;
  uint16_t* dKs;
  uint16_t* dVs;
  float* dKp;           // [P, Hkv, Dqk] fp32 accumulators or null
  float* dVp;
  float* delta;         // workspace [Hq, T]: rowsum(dO * O)
  float* dq_part;       // workspace [S, T, Hq, Dqk] fp32 (S > 1)
  const uint16_t* KTp;  // packed prompt K: [Hkv * Dqk, ppad] (pack.hip layout)
  const uint16_t* KTs;  // packed response K: [Hkv * Dqk, tpad], response i from slot spos[i]
  int64_t ppad, tpad;
  int32_t spos[kMaxResp + 1];
  int32_t splits;
  int32_t ptiles;
  int32_t ptiles_per_split;
  int32_t qtiles;
  int32_t tile0[kMaxResp + 1];
  int32_t ktiles_prompt;          // key tiles of the dK/dV kernel over the prompt (0 in response-only mode)
  int32_t ktile0[kMaxResp + 1];   // first suffix key tile of each response
};

struct AttnPlan {
  int splits, ptiles, ptiles_per_split, qtiles;
  int tile0[kMaxResp + 1];
  int ktiles_prompt;
  int ktile0[kMaxResp + 1];
  int64_t ppad, tpad;           // packed prompt / response key slots (multiples of 64)
  int spos[kMaxResp + 1];       // first packed slot of each response
  size_t ws_bytes;
  size_t off_a, off_b, off_c, off_d;   // workspace sub-buffer offsets
};

// which: 0 fwd, 1 bwd exact, 2 bwd response-only. Returns false if (Dqk, Dv) has no kernel.
bool plan_attn(int which, int P, int Hq, int Hkv, int Dqk, int Dv, int n_resp, const int32_t* cu, AttnPlan* plan);
hipError_t launch_attn_fwd(FwdArgs& a, int Dqk, int Dv, hipStream_t st);
hipError_t launch_attn_bwd(BwdArgs& a, int Dqk, int Dv, hipStream_t st);
// dQ part of the backward (replay_attn_dq.hip): K packing, dQ kernel, split reduction
hipError_t launch_bwd_dq(BwdArgs& a, int Dqk, int Dv, hipStream_t st);

// Kernel timer hooks (timer.cpp): bracket a launch; no-ops unless the timer is armed for `kernel`
// (an ls_kernel_id value).
void timer_mark(int kernel, hipStream_t st, bool end);

}  // namespace lsr
