/*
 * ls_replay.h -- C ABI of liblsreplay: branch-replay attention and the clipped-GRPO
 * token objective for long-context GRPO, on AMD Instinct MI355X (gfx950).
 *
 * Method: LongStraw branch replay, as summarised in the LongStraw study notes
 * (dimensionstp.github.io, "LongStraw" summary). A long prompt's per-layer state
 * (here: one attention layer's K/V) is captured once and kept resident (§2-1 step 1,
 * §3-2 (1)-(2)); the G responses of a group are then replayed one at a time against it,
 * each response's backward adding its prompt-side gradient into resident accumulators
 * (§2-1 step 4, §3-2 (4)), with a single finalisation after the last response (§2-1
 * step 5, §3-2 (7)). The per-token objective is the clipped GRPO policy loss (§1-1,
 * L_policy equation).
 *
 * Conventions for every entry point:
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call only
 *    enqueues work on that stream and returns; it never synchronises.
 *  - Pointers marked "device" are caller-owned device allocations; pointers marked "host"
 *    are read during the call only. The computing entry points allocate no device memory and
 *    keep no state (the optional kernel timer at the end of this header keeps host-side
 *    events while armed).
 *  - bf16 is IEEE bfloat16 stored as 16-bit words; fp32 is IEEE binary32.
 *  - All argument checks run on the host before any HIP call; a failed check returns an
 *    error code and touches no memory. A HIP launch/runtime error returns LS_ERR_HIP.
 *    Nothing throws or aborts across the ABI. NaN/Inf in data propagate and are not checked.
 *  - Results are bitwise reproducible run to run for the same inputs and arguments:
 *    no floating-point atomics are used on any output.
 */
#ifndef LS_REPLAY_H
#define LS_REPLAY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LS_OK = 0,
  LS_ERR_INVALID_ARG = -1, /* a pointer, size, stride or value is invalid                 */
  LS_ERR_UNSUPPORTED = -2, /* valid, but this build has no kernel for it (e.g. head dim)  */
  LS_ERR_WORKSPACE = -3,   /* workspace missing or smaller than ls_*_workspace_bytes      */
  LS_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed                   */
} ls_status;

/* Shape of one attention layer in replay.
 *  P        prompt length (>= 0; 0 gives plain causal attention over the response).
 *  Hq, Hkv  query / key-value heads, Hq % Hkv == 0; query head h reads kv head h / (Hq/Hkv).
 *  Dqk, Dv  head dims; supported pairs: (64,64), (128,128), and (576,512) for latent KV (the
 *           absorbed-latent attention over the GLM run's latent pages, LongStraw study notes §3-1 overview
 *           table and §3-2 (1), (5)).
 *           Other pairs: LS_ERR_UNSUPPORTED.
 *  ldk, ldv elements between consecutive tokens of K and of V, for prompt and suffix alike;
 *           element (token j, kv head k, dim d) sits at K[j*ldk + k*Dqk + d] and
 *           V[j*ldv + k*Dv + d]. ldk >= Hkv*Dqk, ldv >= Hkv*Dv, both multiples of 8.
 *           Latent KV (Hkv == 1, V = first Dv dims of K) passes V = K and ldv = ldk. For
 *           (576,512) this aliasing is required: Hkv must be 1, ldv == ldk, and every call must
 *           pass Vp == Kp (when P > 0) and Vs == Ks; otherwise LS_ERR_UNSUPPORTED (the latent
 *           kernels read V from the K rows and never touch a separate V buffer).
 *  softmax_scale  finite and > 0 (the usual choice is 1/sqrt(Dqk)).
 */
typedef struct ls_attn_desc {
  int32_t P;
  int32_t Hq, Hkv;
  int32_t Dqk, Dv;
  int64_t ldk, ldv;
  float softmax_scale;
} ls_attn_desc;

#define LS_MAX_RESPONSES_PER_CALL 64

/* Workspace size in bytes for ls_replay_attn_fwd (which = 0) or ls_replay_attn_bwd
 * (which = 1, exact prompt-gradient mode; which = 2, response-only mode) with these
 * arguments. cu_seqlens: host, n_resp + 1 packed-row offsets (see ls_replay_attn_fwd).
 * Writes the size to *bytes. Errors: LS_ERR_INVALID_ARG / LS_ERR_UNSUPPORTED as the
 * matching call would return. */
int ls_replay_attn_workspace_bytes(const ls_attn_desc* desc, int32_t n_resp, const int32_t* cu_seqlens,
                                   int32_t which, size_t* bytes);

/* Replay attention forward (LongStraw study notes §2-1 step 4, §3-2 (2) and (4)).
 * n_resp (1..LS_MAX_RESPONSES_PER_CALL) responses are packed along the token axis:
 * response i owns rows cu_seqlens[i] .. cu_seqlens[i+1]-1 (host array, cu_seqlens[0] = 0,
 * non-decreasing; empty responses are allowed). T = cu_seqlens[n_resp].
 * For response i, row t (0-based within the response) and query head h, with k = h/(Hq/Hkv):
 * the query attends to all P prompt keys Kp[:,k] and to the response's own keys Ks[s,k]
 * for s <= t, with softmax over scores softmax_scale * <q, key>.
 *  Kp, Vp  device bf16 [P, Hkv, *] with strides ldk/ldv; READ ONLY (the library never writes
 *          prompt state, so it can be reused for every response of the group, §3-2 (3)).
 *          May be NULL when P == 0.
 *  Q       device bf16 [T, Hq, Dqk] contiguous.
 *  Ks, Vs  device bf16 [T, Hkv, *] with strides ldk/ldv (latent KV: Vs = Ks).
 *  O       device bf16 [T, Hq, Dv] contiguous, overwritten.
 *  lse     device fp32 [Hq, T], overwritten: natural-log sum of exp of the visible scores.
 *  O_lo    optional device bf16 [T, Hq, Dv] contiguous, or NULL. When given it is overwritten with
 *          the bf16 of O32 - O, where O32 is the fp32 output before rounding: O + O_lo carries
 *          the output to about 16 significant bits. The backward uses it for the row term
 *          Delta = rowsum(dO * O) of dS = P (dP - Delta); without it Delta sees O's bf16 rounding,
 *          which matters only where a handful of prompt keys carry whole softmax rows (very
 *          short prompts: the prompt accumulators then drift by ~2e-3 relative instead of <1e-3).
 *  workspace  device, >= ls_replay_attn_workspace_bytes(which = 0), 256-byte aligned; may be
 *          NULL when that size is 0.
 * All device pointers 16-byte aligned. T == 0 returns LS_OK and launches nothing. */
int ls_replay_attn_fwd(void* stream, const ls_attn_desc* desc,
                       const void* Kp, const void* Vp,
                       int32_t n_resp, const int32_t* cu_seqlens,
                       const void* Q, const void* Ks, const void* Vs,
                       void* O, float* lse, void* O_lo,
                       void* workspace, size_t workspace_bytes);

/* Replay attention backward (same section; the prompt-side term is the dl/dz_P part of the
 * gradient decomposition of §2-2). Arguments as in ls_replay_attn_fwd, plus:
 *  O, lse  the forward's outputs for these inputs.
 *  O_lo    the forward's O_lo for these inputs, or NULL (Delta from the bf16 O alone).
 *  dO      device bf16 [T, Hq, Dv] contiguous.
 *  dQ      device bf16 [T, Hq, Dqk] contiguous, overwritten.
 *  dKs     device bf16 [T, Hkv, Dqk] contiguous, overwritten.
 *  dVs     device bf16 [T, Hkv, Dv] contiguous, overwritten (latent KV: returned separately
 *          from dKs; the latent gradient is dKs plus dVs padded to Dqk, formed by the caller).
 *  dKp_accum, dVp_accum  device fp32 [P, Hkv, Dqk] / [P, Hkv, Dv] contiguous. Both non-NULL:
 *          exact prompt-gradient mode, the prompt-side gradient of these responses is ADDED in
 *          place (never zeroed by the library: the caller zeroes them at the start of a group
 *          and reads them after the last response). Both NULL: response-only closure (stop-
 *          gradient prompt boundary, §2-2), accumulators not touched. Exactly one NULL is
 *          LS_ERR_INVALID_ARG. Two calls that add into the same accumulators must be ordered
 *          (same stream or caller events).
 *  workspace  >= ls_replay_attn_workspace_bytes(which = 1 exact, 2 response-only). */
int ls_replay_attn_bwd(void* stream, const ls_attn_desc* desc,
                       const void* Kp, const void* Vp,
                       int32_t n_resp, const int32_t* cu_seqlens,
                       const void* Q, const void* Ks, const void* Vs,
                       const void* O, const float* lse, const void* O_lo, const void* dO,
                       void* dQ, void* dKs, void* dVs,
                       float* dKp_accum, float* dVp_accum,
                       void* workspace, size_t workspace_bytes);

/* Blockwise replay of one long response (LongStraw study notes §3-2, blockwise suffix replay):
 * the response's query rows are replayed in blocks; block rows q0 .. q0+nq-1 attend to all P
 * prompt keys and causally to the response's keys 0 .. q0+nq-1 (their own and every earlier
 * block's), so the blocks together give exactly the full response's attention and gradients.
 *  q0, nq   first row of the block within the response (>= 0) and its rows (>= 0).
 *  Q        device bf16 [nq, Hq, Dqk]: the block's queries.
 *  Ks, Vs   device bf16 [q0 + nq, Hkv, *] with strides ldk/ldv: the response's keys from its
 *           first token through the block's last.
 *  O, lse   device bf16 [nq, Hq, Dv] and fp32 [Hq, nq] for the block's rows, overwritten.
 *  O_lo     optional bf16 [nq, Hq, Dv] rounding residual of O, as in ls_replay_attn_fwd.
 * Other arguments as in ls_replay_attn_fwd. nq == 0 returns LS_OK and launches nothing. */
int ls_replay_attn_block_workspace_bytes(const ls_attn_desc* desc, int32_t q0, int32_t nq, int32_t which,
                                         size_t* bytes);
int ls_replay_attn_fwd_block(void* stream, const ls_attn_desc* desc,
                             const void* Kp, const void* Vp,
                             int32_t q0, int32_t nq,
                             const void* Q, const void* Ks, const void* Vs,
                             void* O, float* lse, void* O_lo,
                             void* workspace, size_t workspace_bytes);

/* Backward of one block (arguments as in ls_replay_attn_fwd_block and ls_replay_attn_bwd):
 *  O, lse, dO  the block's forward outputs and output gradient: [nq, Hq, Dv], [Hq, nq], [nq, Hq, Dv].
 *  O_lo        the block forward's O_lo, or NULL.
 *  dQ          device bf16 [nq, Hq, Dqk], overwritten (the block's rows only).
 *  dKs_accum, dVs_accum  device fp32 [q0 + nq, Hkv, Dqk] / [q0 + nq, Hkv, Dv] contiguous, both
 *              required: the block's contribution to the gradients of the response's keys
 *              0 .. q0+nq-1 is ADDED (the caller zeroes them before the response's first block).
 *  dKp_accum, dVp_accum  prompt accumulators as in ls_replay_attn_bwd (exact mode or both NULL).
 *  workspace   >= ls_replay_attn_block_workspace_bytes(which = 1 exact, 2 response-only).
 * Blocks of one response that add into the same accumulators must be ordered. */
int ls_replay_attn_bwd_block(void* stream, const ls_attn_desc* desc,
                             const void* Kp, const void* Vp,
                             int32_t q0, int32_t nq,
                             const void* Q, const void* Ks, const void* Vs,
                             const void* O, const float* lse, const void* O_lo, const void* dO,
                             void* dQ, float* dKs_accum, float* dVs_accum,
                             float* dKp_accum, float* dVp_accum,
                             void* workspace, size_t workspace_bytes);

/* Workspace bytes for ls_grpo_token_loss over T rows of vocabulary V (written to *bytes). */
int ls_grpo_workspace_bytes(int64_t T, int32_t V, size_t* bytes);

/* Clipped-GRPO token objective and its gradient (LongStraw study notes §1-1, L_policy):
 *   L = -(1/G) sum_i (1/R_i) sum_t min(rho A_i, clip(rho, 1-eps, 1+eps) A_i),
 *   rho = exp(logp - old_logp), logp = log_softmax(logits row)[target],
 *   A_i = (r_i - mean(r)) / (std(r) + 1e-6)  (population std over the G rewards; the
 *   pages say only that the advantage is built from the group rewards).
 * This call handles responses first .. first+count-1, whose rows are packed in `logits`.
 *  V         vocabulary size, 1..2^24 (larger: LS_ERR_UNSUPPORTED). Rows of up to 196608 entries
 *            (V % 8 == 0, 16-byte aligned) are read once; longer rows are read twice.
 *  G, R, rewards  group size and host arrays [G] of all response lengths (each >= 1) and
 *            rewards (finite); A and 1/(G R_i) are formed on the host in float64.
 *  eps       clip range, 0 < eps < 1.
 *  logits    device bf16 [T, V], T = R[first] + ... + R[first+count-1].
 *  targets   device int32 [T], sampled token ids. An id outside [0, V) is not read from
 *            memory: that row's logp, loss term and dlogits become NaN.
 *  old_logp  device fp32 [T].
 *  dlogits   device bf16 [T, V], overwritten with dL/dlogits (may not alias logits), or NULL:
 *            scoring only (log-probs, clip flags and the loss share, no gradient; the logits
 *            are read once and nothing of size V is written).
 *  loss_accum  device fp32 scalar; this call ADDS its share of L (ordered, deterministic).
 *  logp_out  device fp32 [T] or NULL; clipped_out device uint8 [T] or NULL (1 where the
 *            clipped branch is strictly smaller, so the token's gradient is zero).
 *  workspace >= ls_grpo_workspace_bytes(T, V), 16-byte aligned.
 * logits/dlogits rows are read/written with 16-byte accesses when V % 8 == 0 and both are
 * 16-byte aligned, else element-wise. */
int ls_grpo_token_loss(void* stream, int32_t V, int32_t G,
                       const int32_t* R, const float* rewards,
                       float eps, int32_t first, int32_t count,
                       const void* logits, const int32_t* targets, const float* old_logp,
                       void* dlogits, float* loss_accum,
                       float* logp_out, uint8_t* clipped_out,
                       void* workspace, size_t workspace_bytes);

/* ls_grpo_token_loss without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. Arguments,
 * outputs and errors are those of ls_grpo_token_loss, and so are the kernels and every result. The
 * per-row loss terms that the workspace held go to a fixed array of LS_NOALLOC_MAX_ROWS floats
 * (4 MiB) in the library's device memory, one per GPU, held until the process ends. This call
 * allocates no device memory; its first call on a device looks the array's address up (a HIP symbol
 * query; a failure returns LS_ERR_HIP).
 *  Rows per call (the summed R_i of the selected responses) at most LS_NOALLOC_MAX_ROWS; more
 *  returns LS_ERR_WORKSPACE before anything is launched.
 * Every call on one GPU uses that GPU's array and leaves the last call's terms in it. Calls that
 * overlap on one GPU (several streams, or host threads without ordering) race on it: the caller
 * orders them. */
#define LS_NOALLOC_MAX_ROWS 1048576
int ls_grpo_token_loss_noalloc(void* stream, int32_t V, int32_t G,
                               const int32_t* R, const float* rewards,
                               float eps, int32_t first, int32_t count,
                               const void* logits, const int32_t* targets, const float* old_logp,
                               void* dlogits, float* loss_accum,
                               float* logp_out, uint8_t* clipped_out);

/* Workspace bytes for ls_grpo_lmhead_loss over T rows (written to *bytes): for one chunk of at
 * most 4096 tokens (fewer where V > 262144, so that a chunk's [tokens, V] bf16 buffer stays under
 * 2 GiB) the dlogits buffer, the per-slab softmax partials, target logits and per-row loss terms,
 * and the split partials of dH. */
int ls_grpo_lmhead_workspace_bytes(int64_t T, int32_t V, int32_t d, size_t* bytes);

/* LM head fused with the clipped-GRPO token objective: the objective above (LongStraw study notes
 * §1-1, L_policy, over the vocabulary) applied to logits = H W^T, formed chunk by chunk so that a
 * response's [T, V] logits never exist. Per chunk, all on this library's gfx950 kernels:
 *   a GEMM forms the logits in fp32 and, in its epilogue, rounds them to bf16 and reduces them per
 *   token and 128-word vocabulary slab to (max, sum of exp(x - max)) and the target's logit; the
 *   logits are never written to memory. With gradients, the epilogue also stores
 *   e = exp(x - slab max) (bf16) in the workspace's dlogits buffer;
 *   a row kernel merges each token's slab partials into its log-sum-exp, forms the loss share,
 *   log-prob and clip flag as ls_grpo_token_loss does, and rescales the stored e in place into
 *   bf16 dlogits (the one-hot term from the target's logit);
 *   two more GEMMs form dH = dlogits W (bf16, overwritten; split over V, fp32 partials summed in a
 *   fixed order) and dW += dlogits^T H (fp32, added in place).
 * Results are run-to-run identical (fixed summation orders, no atomics). Nothing is allocated.
 * The dlogits differ from ls_grpo_token_loss's on the same logits by the extra bf16 rounding of e.
 *  V, d      vocabulary size (8 .. 2^24, a multiple of 8) and hidden size (8 .. 65536, a multiple
 *            of 8); V * d < 2^31. Other values: LS_ERR_UNSUPPORTED.
 *  G, R, rewards, eps, first, count  as for ls_grpo_token_loss.
 *  H         device bf16 [T, d] hidden states of the selected responses' tokens, packed.
 *  W         device bf16 [V, d] vocabulary projection; read only.
 *  targets, old_logp, loss_accum, logp_out, clipped_out  as for ls_grpo_token_loss.
 *  dH        device bf16 [T, d], overwritten with dL/dH; and
 *  dW_accum  device fp32 [V, d]; this call ADDS dL/dW (the caller zeroes it once per step).
 *            Both NULL: scoring only (no e stores, no gradient GEMMs). Exactly one NULL:
 *            LS_ERR_INVALID_ARG.
 *  workspace >= ls_grpo_lmhead_workspace_bytes(T, V, d), 256-byte aligned.
 * H, W, dH and dW_accum must be 16-byte aligned. The work runs on `stream`; calls that overlap
 * on one device must use separate workspaces. */
int ls_grpo_lmhead_loss(void* stream, int32_t V, int32_t d, int32_t G,
                        const int32_t* R, const float* rewards, float eps,
                        int32_t first, int32_t count,
                        const void* H, const void* W,
                        const int32_t* targets, const float* old_logp,
                        float* loss_accum, void* dH, float* dW_accum,
                        float* logp_out, uint8_t* clipped_out,
                        void* workspace, size_t workspace_bytes);

/* Static string naming a status code. */
const char* ls_status_string(int status);

/* Kernel timer -- instrumentation for benchmarks, not part of the replay computation.
 * ls_kernel_timer_start arms the timer for one kernel and clears earlier records; from then on
 * every launch of that kernel by the entry points above is bracketed by two HIP events recorded
 * on the caller's stream (the events are created by the library on first use and kept for reuse).
 * ls_kernel_timer_stop disarms it, waits for the recorded events and writes the summed device
 * time in milliseconds and the number of launches. At most 65536 launches are recorded per
 * arming (more: stop returns LS_ERR_HIP). Errors: an unknown kernel id, NULL outputs or stop
 * without start give LS_ERR_INVALID_ARG; a failed event call gives LS_ERR_HIP. The timer is
 * process-wide and guarded by a mutex; timing calls on several streams at once is allowed but
 * sums their overlapping durations. */
typedef enum {
  LS_KERNEL_ATTN_FWD = 0,     /* replay attention forward main kernel (split partials)      */
  LS_KERNEL_DKDV_PROMPT = 1,  /* backward dK/dV over the prompt keys (exact mode only)       */
  LS_KERNEL_DQ = 2,           /* backward dQ (split over the prompt keys)                    */
  LS_KERNEL_GRPO_ROWS = 3     /* per-row pass of the GRPO token loss                         */
} ls_kernel_id;

int ls_kernel_timer_start(int32_t kernel);
int ls_kernel_timer_stop(float* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* LS_REPLAY_H */
