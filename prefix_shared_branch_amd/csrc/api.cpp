// Host side of liblsreplay: argument validation (pure C++, before any HIP call),
// workspace sizing, advantage computation and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/ls_replay.h"
#include "kernels.h"

namespace {

using lsr::kMaxResp;
constexpr int32_t kMaxVocab = 1 << 24;  // rows above 196608 stream twice (32-bit element offsets)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_desc(const ls_attn_desc* d) {
  if (!d) return LS_ERR_INVALID_ARG;
  if (d->P < 0 || d->Hq < 1 || d->Hkv < 1 || (d->Hq % d->Hkv) != 0) return LS_ERR_INVALID_ARG;
  if (d->Dqk < 1 || d->Dv < 1 || d->Dv > d->Dqk) return LS_ERR_INVALID_ARG;
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.0f)) return LS_ERR_INVALID_ARG;
  if (d->ldk < (int64_t)d->Hkv * d->Dqk || d->ldv < (int64_t)d->Hkv * d->Dv) return LS_ERR_INVALID_ARG;
  if ((d->ldk % 8) != 0 || (d->ldv % 8) != 0) return LS_ERR_INVALID_ARG;
  const bool wide = d->Dqk == lsr::kWideDqk && d->Dv == lsr::kWideDv;
  const bool ok_shape = (d->Dqk == 64 && d->Dv == 64) || (d->Dqk == 128 && d->Dv == 128) || wide;
  if (!ok_shape) return LS_ERR_UNSUPPORTED;
  // latent KV: one kv head whose V rows are the leading Dv dims of the K rows (same row stride)
  if (wide && (d->Hkv != 1 || d->ldv != d->ldk)) return LS_ERR_UNSUPPORTED;
  return LS_OK;
}

// latent-KV heads: V must alias K (the wide kernels read both from the K rows)
int check_alias(const ls_attn_desc* d, const void* Kp, const void* Vp, const void* Ks, const void* Vs) {
  if (d->Dqk != lsr::kWideDqk) return LS_OK;
  if (Vs != Ks || (d->P > 0 && Vp != Kp)) return LS_ERR_UNSUPPORTED;
  return LS_OK;
}

int check_cu(int32_t n_resp, const int32_t* cu) {
  if (n_resp < 1 || !cu) return LS_ERR_INVALID_ARG;
  if (n_resp > LS_MAX_RESPONSES_PER_CALL) return LS_ERR_UNSUPPORTED;
  if (cu[0] != 0) return LS_ERR_INVALID_ARG;
  for (int i = 0; i < n_resp; ++i)
    if (cu[i + 1] < cu[i]) return LS_ERR_INVALID_ARG;
  return LS_OK;
}

// cu: query-row offsets; kcu: response-key offsets (kcu == cu, or one response whose keys start
// before its first query row)
int plan_for(const ls_attn_desc* d, int32_t n_resp, const int32_t* cu, const int32_t* kcu, int which,
             lsr::AttnPlan* pl) {
  int st = check_desc(d);
  if (st != LS_OK) return st;
  st = check_cu(n_resp, cu);
  if (st != LS_OK) return st;
  // sizes must fit the kernels' 32-bit row arithmetic
  const int64_t T = cu[n_resp];
  const int64_t Tk = kcu[n_resp];
  const int64_t g = d->Hq / d->Hkv;
  if (T * d->Hq > INT32_MAX || T * g > INT32_MAX / 2 || (int64_t)d->P + Tk > INT32_MAX / 2) return LS_ERR_UNSUPPORTED;
  // the backward's packed query-row tiles use 32-bit per-lane offsets: Dqk rows of T * g slots
  if ((T * g + 64) * (int64_t)(d->Dqk > d->Dv ? d->Dqk : d->Dv) * 2 > INT32_MAX) return LS_ERR_UNSUPPORTED;
  if (!lsr::plan_attn(which, d->P, d->Hq, d->Hkv, d->Dqk, d->Dv, n_resp, cu, kcu, pl)) return LS_ERR_UNSUPPORTED;
  return LS_OK;
}

void fill_geom(lsr::AttnGeom* g, const ls_attn_desc* d, const void* Kp, const void* Vp, int32_t n_resp,
               const int32_t* cu, const int32_t* kcu, const void* Q, const void* Ks, const void* Vs) {
  g->Kp = static_cast<const uint16_t*>(Kp);
  g->Vp = static_cast<const uint16_t*>(Vp);
  g->Q = static_cast<const uint16_t*>(Q);
  g->Ks = static_cast<const uint16_t*>(Ks);
  g->Vs = static_cast<const uint16_t*>(Vs);
  g->ldk = d->ldk;
  g->ldv = d->ldv;
  g->P = d->P;
  g->Hq = d->Hq;
  g->Hkv = d->Hkv;
  g->g = d->Hq / d->Hkv;
  g->T = cu[n_resp];
  g->scale = d->softmax_scale;
  g->scale_log2 = d->softmax_scale * 1.4426950408889634f;
  g->n_resp = n_resp;
  for (int i = 0; i <= kMaxResp; ++i) g->tok0[i] = cu[i <= n_resp ? i : n_resp];
  g->Tk = kcu[n_resp];
  for (int i = 0; i <= kMaxResp; ++i) g->ktok0[i] = kcu[i <= n_resp ? i : n_resp];
}

int fwd_impl(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t n_resp,
             const int32_t* cu_seqlens, const int32_t* kcu, const void* Q, const void* Ks, const void* Vs, void* O,
             float* lse, void* O_lo, void* workspace, size_t workspace_bytes);
int bwd_impl(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t n_resp,
             const int32_t* cu_seqlens, const int32_t* kcu, const void* Q, const void* Ks, const void* Vs,
             const void* O, const float* lse, const void* O_lo, const void* dO, void* dQ, void* dKs, void* dVs,
             float* dKs_acc, float* dVs_acc, float* dKp_accum, float* dVp_accum, void* workspace,
             size_t workspace_bytes);

}  // namespace

extern "C" {

const char* ls_status_string(int status) {
  switch (status) {
    case LS_OK: return "LS_OK";
    case LS_ERR_INVALID_ARG: return "LS_ERR_INVALID_ARG";
    case LS_ERR_UNSUPPORTED: return "LS_ERR_UNSUPPORTED";
    case LS_ERR_WORKSPACE: return "LS_ERR_WORKSPACE";
    case LS_ERR_HIP: return "LS_ERR_HIP";
    default: return "LS_UNKNOWN_STATUS";
  }
}

int ls_replay_attn_workspace_bytes(const ls_attn_desc* desc, int32_t n_resp, const int32_t* cu_seqlens,
                                   int32_t which, size_t* bytes) {
  if (!bytes || which < 0 || which > 2) return LS_ERR_INVALID_ARG;
  lsr::AttnPlan pl;
  const int st = plan_for(desc, n_resp, cu_seqlens, cu_seqlens, which, &pl);
  if (st != LS_OK) return st;
  *bytes = pl.ws_bytes;
  return LS_OK;
}

int ls_replay_attn_fwd(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t n_resp,
                       const int32_t* cu_seqlens, const void* Q, const void* Ks, const void* Vs, void* O, float* lse,
                       void* O_lo, void* workspace, size_t workspace_bytes) {
  return fwd_impl(stream, desc, Kp, Vp, n_resp, cu_seqlens, cu_seqlens, Q, Ks, Vs, O, lse, O_lo, workspace,
                  workspace_bytes);
}

int ls_replay_attn_bwd(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t n_resp,
                       const int32_t* cu_seqlens, const void* Q, const void* Ks, const void* Vs, const void* O,
                       const float* lse, const void* O_lo, const void* dO, void* dQ, void* dKs, void* dVs,
                       float* dKp_accum, float* dVp_accum, void* workspace, size_t workspace_bytes) {
  if (!dKs || !dVs) return LS_ERR_INVALID_ARG;
  return bwd_impl(stream, desc, Kp, Vp, n_resp, cu_seqlens, cu_seqlens, Q, Ks, Vs, O, lse, O_lo, dO, dQ, dKs, dVs,
                  nullptr, nullptr, dKp_accum, dVp_accum, workspace, workspace_bytes);
}

int ls_replay_attn_block_workspace_bytes(const ls_attn_desc* desc, int32_t q0, int32_t nq, int32_t which,
                                         size_t* bytes) {
  if (!bytes || which < 0 || which > 2 || q0 < 0 || nq < 0 || (int64_t)q0 + nq > INT32_MAX) return LS_ERR_INVALID_ARG;
  const int32_t cu[2] = {0, nq}, kcu[2] = {0, q0 + nq};
  lsr::AttnPlan pl;
  const int st = plan_for(desc, 1, cu, kcu, which, &pl);
  if (st != LS_OK) return st;
  *bytes = pl.ws_bytes;
  return LS_OK;
}

int ls_replay_attn_fwd_block(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t q0,
                             int32_t nq, const void* Q, const void* Ks, const void* Vs, void* O, float* lse, void* O_lo,
                             void* workspace, size_t workspace_bytes) {
  if (q0 < 0 || nq < 0 || (int64_t)q0 + nq > INT32_MAX) return LS_ERR_INVALID_ARG;
  const int32_t cu[2] = {0, nq}, kcu[2] = {0, q0 + nq};
  return fwd_impl(stream, desc, Kp, Vp, 1, cu, kcu, Q, Ks, Vs, O, lse, O_lo, workspace, workspace_bytes);
}

int ls_replay_attn_bwd_block(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t q0,
                             int32_t nq, const void* Q, const void* Ks, const void* Vs, const void* O,
                             const float* lse, const void* O_lo, const void* dO, void* dQ, float* dKs_accum,
                             float* dVs_accum, float* dKp_accum, float* dVp_accum, void* workspace,
                             size_t workspace_bytes) {
  if (q0 < 0 || nq < 0 || (int64_t)q0 + nq > INT32_MAX) return LS_ERR_INVALID_ARG;
  if (!dKs_accum || !dVs_accum) return LS_ERR_INVALID_ARG;
  const int32_t cu[2] = {0, nq}, kcu[2] = {0, q0 + nq};
  return bwd_impl(stream, desc, Kp, Vp, 1, cu, kcu, Q, Ks, Vs, O, lse, O_lo, dO, dQ, nullptr, nullptr, dKs_accum,
                  dVs_accum, dKp_accum, dVp_accum, workspace, workspace_bytes);
}

}  // extern "C"

namespace {

int fwd_impl(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t n_resp,
             const int32_t* cu_seqlens, const int32_t* kcu, const void* Q, const void* Ks, const void* Vs, void* O,
             float* lse, void* O_lo, void* workspace, size_t workspace_bytes) {
  lsr::AttnPlan pl;
  int st = plan_for(desc, n_resp, cu_seqlens, kcu, 0, &pl);
  if (st != LS_OK) return st;
  const int64_t T = cu_seqlens[n_resp];
  if (desc->P > 0 && (!Kp || !Vp || !aligned(Kp, 16) || !aligned(Vp, 16))) return LS_ERR_INVALID_ARG;
  if ((st = check_alias(desc, Kp, Vp, Ks, Vs)) != LS_OK) return st;
  if (T == 0) return LS_OK;
  const void* dev[] = {Q, Ks, Vs, O, lse};
  for (const void* p : dev)
    if (!p || !aligned(p, 16)) return LS_ERR_INVALID_ARG;
  if (O_lo && !aligned(O_lo, 16)) return LS_ERR_INVALID_ARG;
  if (pl.ws_bytes > 0 && (!workspace || !aligned(workspace, 256))) return LS_ERR_WORKSPACE;
  if (workspace_bytes < pl.ws_bytes) return LS_ERR_WORKSPACE;

  lsr::FwdArgs a;
  std::memset(&a, 0, sizeof(a));
  fill_geom(&a.geo, desc, Kp, Vp, n_resp, cu_seqlens, kcu, Q, Ks, Vs);
  a.O = static_cast<uint16_t*>(O);
  a.O_lo = static_cast<uint16_t*>(O_lo);
  a.lse = lse;
  char* ws = static_cast<char*>(workspace);
  a.o_part = pl.splits > 1 ? reinterpret_cast<float*>(ws + pl.off_a) : nullptr;
  a.lse_part = pl.splits > 1 ? reinterpret_cast<float*>(ws + pl.off_b) : nullptr;
  a.splits = pl.splits;
  a.ptiles = pl.ptiles;
  a.ptiles_per_split = pl.ptiles_per_split;
  a.qtiles = pl.qtiles;
  for (int i = 0; i <= kMaxResp; ++i) a.tile0[i] = pl.tile0[i];
  a.VTp = reinterpret_cast<const uint16_t*>(ws + pl.off_c);
  a.VTs = reinterpret_cast<const uint16_t*>(ws + pl.off_d);
  if (desc->Dqk != lsr::kWideDqk) {  // latent KV reads V from the K tiles as bf16 (no V scale)
    a.vscale_part = reinterpret_cast<float*>(ws + pl.off_sc);
    a.vscale = a.vscale_part + lsr::kScaleBlocks * 8;
  }
  a.ppad = pl.ppad;
  a.tpad = pl.tpad;
  for (int i = 0; i <= kMaxResp; ++i) a.spos[i] = pl.spos[i];
  const hipError_t e = lsr::launch_attn_fwd(a, desc->Dqk, desc->Dv, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LS_OK : LS_ERR_HIP;
}

int bwd_impl(void* stream, const ls_attn_desc* desc, const void* Kp, const void* Vp, int32_t n_resp,
             const int32_t* cu_seqlens, const int32_t* kcu, const void* Q, const void* Ks, const void* Vs,
             const void* O, const float* lse, const void* O_lo, const void* dO, void* dQ, void* dKs, void* dVs,
             float* dKs_acc, float* dVs_acc, float* dKp_accum, float* dVp_accum, void* workspace,
             size_t workspace_bytes) {
  if ((dKp_accum == nullptr) != (dVp_accum == nullptr)) return LS_ERR_INVALID_ARG;
  const bool exact = dKp_accum != nullptr;
  lsr::AttnPlan pl;
  int st = plan_for(desc, n_resp, cu_seqlens, kcu, exact ? 1 : 2, &pl);
  if (st != LS_OK) return st;
  const int64_t T = cu_seqlens[n_resp];
  if (desc->P > 0 && (!Kp || !Vp || !aligned(Kp, 16) || !aligned(Vp, 16))) return LS_ERR_INVALID_ARG;
  if (exact && desc->P > 0 && (!aligned(dKp_accum, 16) || !aligned(dVp_accum, 16))) return LS_ERR_INVALID_ARG;
  if ((st = check_alias(desc, Kp, Vp, Ks, Vs)) != LS_OK) return st;
  if (T == 0) return LS_OK;
  const void* dev[] = {Q, Ks, Vs, O, lse, dO, dQ, dKs_acc ? dKs_acc : dKs, dVs_acc ? dVs_acc : dVs};
  for (const void* p : dev)
    if (!p || !aligned(p, 16)) return LS_ERR_INVALID_ARG;
  if (O_lo && !aligned(O_lo, 16)) return LS_ERR_INVALID_ARG;
  if (pl.ws_bytes > 0 && (!workspace || !aligned(workspace, 256))) return LS_ERR_WORKSPACE;
  if (workspace_bytes < pl.ws_bytes) return LS_ERR_WORKSPACE;

  lsr::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  fill_geom(&a.geo, desc, Kp, Vp, n_resp, cu_seqlens, kcu, Q, Ks, Vs);
  a.O = static_cast<const uint16_t*>(O);
  a.O_lo = static_cast<const uint16_t*>(O_lo);
  a.lse = lse;
  a.dO = static_cast<const uint16_t*>(dO);
  a.dQ = static_cast<uint16_t*>(dQ);
  a.dKs = static_cast<uint16_t*>(dKs);
  a.dVs = static_cast<uint16_t*>(dVs);
  a.dKs_acc = dKs_acc;
  a.dVs_acc = dVs_acc;
  a.dKp = exact && desc->P > 0 ? dKp_accum : nullptr;
  a.dVp = exact && desc->P > 0 ? dVp_accum : nullptr;
  char* ws = static_cast<char*>(workspace);
  a.delta = reinterpret_cast<float*>(ws + pl.off_a);
  a.dq_part = pl.splits > 1 ? reinterpret_cast<float*>(ws + pl.off_b) : nullptr;
  a.splits = pl.splits;
  a.ptiles = pl.ptiles;
  a.ptiles_per_split = pl.ptiles_per_split;
  a.qtiles = pl.qtiles;
  for (int i = 0; i <= kMaxResp; ++i) a.tile0[i] = pl.tile0[i];
  a.Qr = reinterpret_cast<uint16_t*>(ws + pl.off_qr);
  a.dOr = reinterpret_cast<uint16_t*>(ws + pl.off_or);
  a.QT = reinterpret_cast<uint16_t*>(ws + pl.off_qt);
  a.dOT = reinterpret_cast<uint16_t*>(ws + pl.off_ot);
  a.rowstat = reinterpret_cast<float*>(ws + pl.off_rs);
  a.mpad = pl.mpad;
  a.scale_part = reinterpret_cast<float*>(ws + pl.off_sc);
  a.scales = a.scale_part + lsr::kScaleBlocks * 8;
  a.KTp = reinterpret_cast<const uint16_t*>(ws + pl.off_c);
  a.KTs = reinterpret_cast<const uint16_t*>(ws + pl.off_d);
  a.ppad = pl.ppad;
  a.tpad = pl.tpad;
  for (int i = 0; i <= kMaxResp; ++i) a.spos[i] = pl.spos[i];
  a.ktiles_prompt = (a.dKp != nullptr) ? pl.ktiles_prompt : 0;
  for (int i = 0; i <= kMaxResp; ++i) a.ktile0[i] = pl.ktile0[i];
  const hipError_t e = lsr::launch_attn_bwd(a, desc->Dqk, desc->Dv, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LS_OK : LS_ERR_HIP;
}

}  // namespace

namespace lsr {

// one fp32 loss term per row, summed in a fixed order by grpo_sum
size_t grpo_workspace_bytes(int64_t T) { return (size_t)((T * 4 + 255) / 256 * 256); }

bool grpo_batches(int32_t G, const int32_t* R, const float* rewards, float eps, int32_t first, int32_t count,
                  int64_t lo, int64_t hi, const std::function<bool(GrpoArgs&, int64_t)>& fn) {
  // group advantage in float64 on the host: A_i = (r_i - mean) / (std_pop + 1e-6)
  double mean = 0.0;
  for (int i = 0; i < G; ++i) mean += rewards[i];
  mean /= G;
  double var = 0.0;
  for (int i = 0; i < G; ++i) var += (rewards[i] - mean) * (rewards[i] - mean);
  const double sd = std::sqrt(var / G);

  // the rows of each response that fall in [lo, hi), in batches of at most kMaxResp responses
  GrpoArgs a;
  int nb = 0;
  int64_t brow0 = 0, rows = 0;
  auto flush = [&]() -> bool {
    if (nb == 0) return true;
    a.n = nb;
    a.T = rows;
    a.eps = eps;
    nb = 0;
    rows = 0;
    return fn(a, brow0);
  };
  int64_t start = 0;
  for (int i = first; i < first + count; ++i) {
    const int64_t s = start > lo ? start : lo;
    const int64_t e = (start + R[i]) < hi ? (start + R[i]) : hi;
    start += R[i];
    if (s >= e) continue;
    if (nb == 0) {
      std::memset(&a, 0, sizeof(a));
      brow0 = s;
    }
    rows += e - s;
    a.row_end[nb] = (int32_t)rows;
    a.A[nb] = (float)((rewards[i] - mean) / (sd + 1e-6));
    a.w[nb] = (float)(1.0 / ((double)G * (double)R[i]));
    if (++nb == kMaxResp && !flush()) return false;
  }
  return flush();
}

int grpo_rows(hipStream_t st, int32_t V, int32_t G, const int32_t* R, const float* rewards, float eps, int32_t first,
              int32_t count, int64_t lo, int64_t hi, const uint16_t* logits, const int32_t* targets,
              const float* old_logp, uint16_t* dlogits, float* loss_accum, float* logp_out, uint8_t* clipped_out,
              float* row_loss, bool vec) {
  const bool ok = grpo_batches(G, R, rewards, eps, first, count, lo, hi, [&](GrpoArgs& a, int64_t brow0) {
    a.V = V;
    a.logits = logits + (brow0 - lo) * V;
    a.dlogits = dlogits ? dlogits + (brow0 - lo) * V : nullptr;
    a.targets = targets + brow0;
    a.old_logp = old_logp + brow0;
    a.row_loss = row_loss + (brow0 - lo);
    a.logp_out = logp_out ? logp_out + brow0 : nullptr;
    a.clipped_out = clipped_out ? clipped_out + brow0 : nullptr;
    a.loss_accum = loss_accum;
    return launch_grpo(a, vec, st) == hipSuccess;
  });
  return ok ? LS_OK : LS_ERR_HIP;
}

}  // namespace lsr

extern "C" {

int ls_grpo_workspace_bytes(int64_t T, int32_t V, size_t* bytes) {
  if (!bytes || T < 0 || V < 1) return LS_ERR_INVALID_ARG;
  *bytes = lsr::grpo_workspace_bytes(T);
  return LS_OK;
}

int ls_grpo_token_loss(void* stream, int32_t V, int32_t G, const int32_t* R, const float* rewards, float eps,
                       int32_t first, int32_t count, const void* logits, const int32_t* targets,
                       const float* old_logp, void* dlogits, float* loss_accum, float* logp_out,
                       uint8_t* clipped_out, void* workspace, size_t workspace_bytes) {
  if (V < 1 || G < 1 || !R || !rewards) return LS_ERR_INVALID_ARG;
  if (V > kMaxVocab) return LS_ERR_UNSUPPORTED;
  if (!std::isfinite(eps) || !(eps > 0.0f) || !(eps < 1.0f)) return LS_ERR_INVALID_ARG;
  if (first < 0 || count < 1 || (int64_t)first + count > G) return LS_ERR_INVALID_ARG;
  for (int i = 0; i < G; ++i)
    if (R[i] < 1 || !std::isfinite(rewards[i])) return LS_ERR_INVALID_ARG;
  int64_t T = 0;
  for (int i = first; i < first + count; ++i) T += R[i];
  if (T > INT32_MAX) return LS_ERR_UNSUPPORTED;
  if (!logits || !targets || !old_logp || !loss_accum) return LS_ERR_INVALID_ARG;
  if (!aligned(logits, 2) || (dlogits && !aligned(dlogits, 2)) || !aligned(targets, 4) || !aligned(old_logp, 4) ||
      !aligned(loss_accum, 4) || (logp_out && !aligned(logp_out, 4)))
    return LS_ERR_INVALID_ARG;
  if (dlogits) {  // dlogits may not alias logits
    const char* lb = static_cast<const char*>(logits);
    const char* db = static_cast<const char*>(dlogits);
    const int64_t nbytes = T * (int64_t)V * 2;
    if (lb < db + nbytes && db < lb + nbytes) return LS_ERR_INVALID_ARG;
  }
  const size_t need = lsr::grpo_workspace_bytes(T);
  if (!workspace || !aligned(workspace, 16)) return LS_ERR_WORKSPACE;
  if (workspace_bytes < need) return LS_ERR_WORKSPACE;

  const bool vec = (V % 8) == 0 && aligned(logits, 16) && (!dlogits || aligned(dlogits, 16));
  return lsr::grpo_rows(static_cast<hipStream_t>(stream), V, G, R, rewards, eps, first, count, 0, T,
                        static_cast<const uint16_t*>(logits), targets, old_logp, static_cast<uint16_t*>(dlogits),
                        loss_accum, logp_out, clipped_out, static_cast<float*>(workspace), vec);
}

}  // extern "C"
