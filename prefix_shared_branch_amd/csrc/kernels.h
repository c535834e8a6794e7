// Internal launch interface between the host API (api.cpp) and the gfx950 kernels.
// Host code validates every argument before calling these; the launchers assume valid input.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <functional>

#include "../../include/ls_replay.h"

namespace lsr {

constexpr int kMaxResp = 64;
// packed query rows per workgroup of the forward and dQ kernels (the plan's query tiles)
constexpr int kQTileFwd = 256;
constexpr int kQTileDq = 256;
// latent-KV heads (V = the leading kWideDv dims of each K row, one kv head): wide kernels
constexpr int kWideDqk = 576;
constexpr int kWideDv = 512;
constexpr int kQTileFwdWide = 128;
constexpr int kQTileDqWide = 64;
constexpr int kDKTileWide = 64;   // keys per dK/dV workgroup

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
// Row pass of the LM head fused with the loss (grpo_loss.hip): per row, the slab partials of the
// logits GEMM merged into the log-sum-exp, the row's loss term, log-prob and clip flag, and (when
// g.dlogits is set) the row's stored e = exp(x - slab max) turned into bf16 dlogits in place; then
// the fixed-order loss sum. g.logits is unused.
struct LmRowArgs {
  GrpoArgs g;
  const float2* part;  // [T][nslab]: (max, sum exp(x - max)) of each 128-word vocabulary slab
  int32_t nslab;
  const float* xtgt;   // [T] the target's logit
};
hipError_t launch_lm_rows(const LmRowArgs& a, hipStream_t st);
// Host side (api.cpp): the rows of responses first .. first+count-1 that fall in the packed range
// [lo, hi), in batches of at most kMaxResp responses. For each batch, fn(a, brow0) gets a with n, T
// (the batch's rows), eps, row_end, A and w filled in (everything else zero) and the batch's first
// packed row. The advantages come from all G rewards. Returns false as soon as fn does.
bool grpo_batches(int32_t G, const int32_t* R, const float* rewards, float eps, int32_t first, int32_t count,
                  int64_t lo, int64_t hi, const std::function<bool(GrpoArgs&, int64_t)>& fn);
// Loss over the packed rows [lo, hi) of responses first .. first+count-1 (host side, api.cpp): the
// advantages come from all G rewards; `logits`, `dlogits` (or null) and `row_loss` point at row lo,
// targets / old_logp / logp_out / clipped_out at row 0. Returns an ls_status code.
int grpo_rows(hipStream_t st, int32_t V, int32_t G, const int32_t* R, const float* rewards, float eps, int32_t first,
              int32_t count, int64_t lo, int64_t hi, const uint16_t* logits, const int32_t* targets,
              const float* old_logp, uint16_t* dlogits, float* loss_accum, float* logp_out, uint8_t* clipped_out,
              float* row_loss, bool vec);

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
  int32_t tok0[kMaxResp + 1];   // cu_seqlens: query rows of response i are tok0[i] .. tok0[i+1]-1
  // Response keys: rows ktok0[i] .. ktok0[i+1]-1 of Ks / Vs (Tk rows in all). A response has at
  // least as many keys as query rows; query row t sits at key position t + (keys - rows), so a
  // block of a response (its later rows) sees the keys of the earlier rows too.
  int32_t Tk;
  int32_t ktok0[kMaxResp + 1];
};

// Repacking of per-token rows (pack.hip). Logical row r of head h, dim d is read from
//   src[(r / grp) * ld + (r % grp) * gstride + h * hstride + d]
// (K or V rows: grp = 1, hstride = dim; GQA-packed query rows r = t * g + j of kv head h:
// grp = g, ld = Hq * dim, gstride = dim, hstride = g * dim).
struct PackArgs {
  const float* f16_scale;  // null: bf16 copy; else fp16 output of value * (*f16_scale)
  const uint16_t* src;   // bf16
  int64_t ld;
  int32_t grp;
  int64_t gstride, hstride;
  int32_t dim, heads;    // dim a multiple of 64
  int32_t nseg;          // 1 .. kMaxResp segments
  int64_t row0[kMaxResp];  // first source row of each segment
  int32_t n[kMaxResp];     // keys of each segment
  int64_t col0[kMaxResp];  // first output slot of each segment (multiple of 64, increasing)
  uint16_t* out;         // [heads * dim, out_ld] bf16
  int64_t out_ld;        // slots per output row (multiple of 64)
  int64_t cols;          // slots written per row (= out_ld)
};
// dimension-major, slot-permuted: out[(h * dim + d) * out_ld + col0_s + p] (see pack.hip)
hipError_t launch_pack_keys_t(const PackArgs& a, hipStream_t st);
// row-major: out[(h * out_ld + col0_s + r) * dim + d], zero rows past each segment's n_s rows
hipError_t launch_pack_rows(const PackArgs& a, hipStream_t st);
// per packed query row: {LSE * log2 e, Delta} as two floats; padding rows get {+inf, 0}
struct RowStatArgs {
  const float* lse;      // [Hq, T]
  const float* delta;    // [Hq, T]
  const float* scales;   // BwdScales (Delta is stored multiplied by the dS scale)
  float* out;            // pack_rowstats: [Hkv, mpad, 2]; pack_rowext: [Hkv, mpad, 8] (32 bytes per row)
  int32_t T, Hq, g, Hkv;
  int64_t M, mpad;       // packed rows per kv head (T * g) and their padded count
  float c2;              // softmax scale * log2(e) (pack_rowext)
};
hipError_t launch_pack_rowstats(const RowStatArgs& a, hipStream_t st);
// Row terms of the D = 64 / 128 dK/dV kernel as MFMA operands: x = -(LSE log2 e - 15) /
// (scale log2 e) and d = -Delta of each packed row, each split into three bf16 parts whose sum is
// the fp32 value to about 24 significant bits, stored as [hi, mid, lo, 0]. Per block of 32 rows
// (1 KB): the x parts of rows 0..31, 256 zero bytes, the d parts, 256 zero bytes. A 32x32x8 product
// of these rows (k = 0..3, zeros for k = 4..7) with a constant [1, 1, 1, 0] operand starts the S and
// dP accumulators at x and d.
hipError_t launch_pack_rowext(const RowStatArgs& a, hipStream_t st);

// Power-of-two scales of the fp16 operands of the dK/dV products (pack.hip), in device memory:
//   [0] s_dO: dO * s_dO has |values| <= 2^15      [1] s_Q: Q * s_Q has |values| <= 2^15
//   [2] s_dS: 2^15 P (dP - Delta) * s_dS has |values| <= 2^15, from the bound
//       |dP - Delta| <= 2 max_r |dO_r| max_j |V_j|  (Euclidean row norms)
//   [3] s_K (latent-KV heads only): K * s_K has |values| <= 2^15
// Partial maxima are kept as [kScaleBlocks, 8] floats, the scales right after them.
constexpr int kScaleBlocks = 512;
struct ScaleArgs {
  const uint16_t* dO;    // [T, Hq, Dv]
  const uint16_t* Q;     // [T, Hq, Dqk]
  const uint16_t* Vp;    // prompt V rows (stride ldv), may be null when P == 0
  const uint16_t* Vs;    // response V rows (stride ldv)
  int64_t ldv;
  int64_t T, P;
  int64_t Tk;            // response V rows
  int32_t Hq, Hkv, Dqk, Dv;
  float* partial;        // [kScaleBlocks, 8] (the first 4 of each block used here)
  float* scales;         // [4]
};
hipError_t launch_bwd_scales(const ScaleArgs& a, hipStream_t st);
// Forward V scale (head dims 64 / 128): scales[0] = s_V, a power of two with max |V| s_V <= 2^15 over
// the prompt and response V rows, scales[1] = 1 / s_V. Only Vp, Vs, ldv, P, Tk, Hkv, Dv, partial and
// scales are read.
hipError_t launch_fwd_vscale(const ScaleArgs& a, hipStream_t st);

struct FwdArgs {
  AttnGeom geo;
  uint16_t* O;          // bf16 [T, Hq, Dv]
  uint16_t* O_lo;       // optional bf16 [T, Hq, Dv]: bf16 of O - bf16(O), the fp32 output's rounding residual
  float* lse;           // [Hq, T]
  float* o_part;        // [S, T, Hq, Dv] fp32 (S > 1)
  float* lse_part;      // [S, Hq, T] (S > 1)
  const uint16_t* VTp;  // packed prompt V: [Hkv * Dv, ppad] (pack.hip layout)
  const uint16_t* VTs;  // packed response V: [Hkv * Dv, tpad], response i from slot spos[i]
                        // (head dims 64 / 128: fp16 of V s_V, see vscale)
  float* vscale_part;   // [kScaleBlocks, 8] partial maxima of |V|
  float* vscale;        // {s_V, 1 / s_V}
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
  const uint16_t* O_lo;  // optional: the forward's rounding residual of O (Delta from O + O_lo)
  const float* lse;
  const uint16_t* dO;
  uint16_t* dQ;
  uint16_t* dKs;         // bf16 response-key gradients (overwritten), or null with dKs_acc
  uint16_t* dVs;
  float* dKs_acc;       // or fp32 [Tk, Hkv, Dqk] / [Tk, Hkv, Dv] accumulators the response-key
  float* dVs_acc;       //   gradients are added into (blocks of one response)
  float* dKp;           // [P, Hkv, Dqk] fp32 accumulators or null
  float* dVp;
  float* delta;         // workspace [Hq, T]: rowsum(dO * O)
  float* dq_part;       // workspace [S, T, Hq, Dqk] fp32 (S > 1)
  uint16_t* Qr;         // packed query rows per kv head, row-major: [Hkv, mpad, Dqk]
  uint16_t* dOr;        // [Hkv, mpad, Dv]
  uint16_t* QT;         // dimension-major, slot-permuted: [Hkv * Dqk, mpad]
  uint16_t* dOT;        // [Hkv * Dv, mpad]
  float* rowstat;       // latent KV: [Hkv, mpad, 2] {LSE log2 e - 15, Delta * s_dS}; D = 64 / 128:
                        // [Hkv, mpad, 8], the bf16 row terms of pack_rowext
  float* scale_part;    // [kScaleBlocks, 8] partial maxima
  float* scales;        // [4] fp16 operand scales (see ScaleArgs)
  int64_t mpad;         // packed query rows per kv head (T * g) rounded up to 64
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
  int64_t mpad;                 // packed query rows per kv head, rounded up to 64
  size_t ws_bytes;
  size_t off_a, off_b, off_c, off_d;   // workspace sub-buffer offsets
  size_t off_qr, off_or, off_qt, off_ot, off_rs, off_sc;
};

// which: 0 fwd, 1 bwd exact, 2 bwd response-only. Returns false if (Dqk, Dv) has no kernel.
// cu: query-row offsets per response; kcu: response-key offsets (kcu = cu except for a block of a
// response, whose keys start before its first query)
bool plan_attn(int which, int P, int Hq, int Hkv, int Dqk, int Dv, int n_resp, const int32_t* cu, const int32_t* kcu,
               AttnPlan* plan);
hipError_t launch_attn_fwd(FwdArgs& a, int Dqk, int Dv, hipStream_t st);
// latent-KV forward main kernel (replay_attn_wide_fwd.hip); the caller merges split partials
hipError_t launch_attn_fwd_wide(FwdArgs& a, hipStream_t st);
hipError_t launch_attn_bwd(BwdArgs& a, int Dqk, int Dv, hipStream_t st);
// dQ part of the backward (replay_attn_dq.hip): K packing, dQ kernel, split reduction
hipError_t launch_bwd_dq(BwdArgs& a, int Dqk, int Dv, hipStream_t st);
// latent-KV dQ and dK/dV parts (replay_attn_wide_bwd.hip). The dQ launcher leaves split partials
// unreduced (the caller reduces); the dK/dV launcher runs its own scales and packing.
hipError_t launch_bwd_dq_wide(BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dkdv_wide(BwdArgs& a, hipStream_t st);
// dK/dV part (replay_attn_dkdv.hip): query-row packing, prompt and response dK/dV kernels
hipError_t launch_bwd_dkdv(BwdArgs& a, int Dqk, int Dv, hipStream_t st);
// prompt-key dK/dV at head dim 128 with 64 keys per wave (replay_attn_dkdv64.hip); same arguments and
// results as the prompt launch of launch_bwd_dkdv, after the same packing
hipError_t launch_dkdv_prompt_w64(BwdArgs& a, hipStream_t st);

// Kernel timer hooks (timer.cpp): bracket a launch; no-ops unless the timer is armed for `kernel`
// (an ls_kernel_id value).
void timer_mark(int kernel, hipStream_t st, bool end);

}  // namespace lsr
