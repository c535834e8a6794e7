// Work decomposition of replay attention (host side, pure C++).
//
// Query side (forward and dQ kernels): the rows of one kv head are GQA-packed (all g query
// heads of a token are consecutive rows) and cut into tiles of kQTile rows per response.
// Key side: the P prompt keys are cut into tiles of kKTile keys and distributed over S
// splits; the response's own (causal) keys are handled by the last split. Split partials
// are merged by log-sum-exp (forward) or summed (dQ), which is the same algebra as merging
// attention partials of prompt pages held by different owners (LongStraw study notes,
// §3-2 (2): cross-rank log-sum-exp and output merge). S is chosen to fill the chip.
//
// dK/dV kernel: one workgroup owns a tile of keys of one kv head, for every prompt key tile
// (exact prompt-gradient mode only) and every response's suffix key tile.
#include <algorithm>
#include <cstring>

#include "kernels.h"

namespace lsr {

namespace {
constexpr int kKTile = 64;    // keys per forward / dQ tile
constexpr int kDKTilePrompt = 256;  // keys per dK/dV workgroup over the prompt at head dim 128
                                    // (64: kDKTileResp; latent-KV heads: kDKTileWide)
constexpr int kDKTileResp = 128;    // keys per dK/dV workgroup over a response's own keys
constexpr int kTargetBlocks = 2048;
constexpr int kMinTilesPerSplit = 8;
constexpr int kMaxSplits = 64;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

bool plan_attn(int which, int P, int Hq, int Hkv, int Dqk, int Dv, int n_resp, const int32_t* cu, const int32_t* kcu,
               AttnPlan* pl) {
  const bool wide = Dqk == kWideDqk && Dv == kWideDv && Hkv == 1;
  const bool ok = (Dqk == 64 && Dv == 64) || (Dqk == 128 && Dv == 128) || wide;
  if (!ok) return false;
  std::memset(pl, 0, sizeof(*pl));
  const int g = Hq / Hkv;
  const long long T = cu[n_resp];
  const int kQTile = wide ? (which == 0 ? kQTileFwdWide : kQTileDqWide) : (which == 0 ? kQTileFwd : kQTileDq);
  const int kDKTileP = wide ? kDKTileWide : (Dqk == 128 ? kDKTilePrompt : kDKTileResp);
  const int kDKTileR = wide ? kDKTileWide : kDKTileResp;
  int qt = 0, kt = 0, sp = 0;
  for (int i = 0; i < n_resp; ++i) {
    pl->tile0[i] = qt;
    pl->ktile0[i] = kt;
    pl->spos[i] = sp;
    const long long R = cu[i + 1] - cu[i];     // query rows
    const long long Rk = kcu[i + 1] - kcu[i];  // response keys (>= R: a block's keys start earlier)
    qt += (int)((R * g + kQTile - 1) / kQTile);
    kt += (int)((Rk + kDKTileR - 1) / kDKTileR);
    sp += (int)((Rk + kKTile - 1) / kKTile * kKTile);
  }
  for (int i = n_resp; i <= kMaxResp; ++i) {
    pl->tile0[i] = qt;
    pl->ktile0[i] = kt;
    pl->spos[i] = sp;
  }
  pl->ppad = (int64_t)(P + kKTile - 1) / kKTile * kKTile;
  pl->tpad = sp;
  pl->qtiles = qt;
  pl->ptiles = (P + kKTile - 1) / kKTile;
  pl->ktiles_prompt = which == 1 ? (P + kDKTileP - 1) / kDKTileP : 0;

  int S = 1;
  const long long w0 = (long long)qt * Hkv;
  if (pl->ptiles > 0 && w0 > 0) {
    S = (int)std::min<long long>(kMaxSplits, (kTargetBlocks + w0 - 1) / w0);
    S = std::max(1, std::min(S, pl->ptiles / kMinTilesPerSplit));
  }
  int pps = pl->ptiles > 0 ? (pl->ptiles + S - 1) / S : 0;
  if (pps > 0) S = (pl->ptiles + pps - 1) / pps;  // no empty splits
  pl->splits = S;
  pl->ptiles_per_split = pps;

  size_t off = 0;
  if (which == 0) {
    if (S > 1) {
      pl->off_a = off;
      off = align256(off + (size_t)S * T * Hq * Dv * 4);
      pl->off_b = off;
      off = align256(off + (size_t)S * Hq * T * 4);
    }
    // dimension-major packed V of the prompt and of the responses (latent KV: read from the K tiles)
    if (!wide) {
      pl->off_c = off;
      off = align256(off + (size_t)Hkv * Dv * pl->ppad * 2);
      pl->off_d = off;
      off = align256(off + (size_t)Hkv * Dv * pl->tpad * 2);
      pl->off_sc = off;  // fp16 scale of V: partial maxima (8 per block), then the scale
      off = align256(off + (size_t)(kScaleBlocks + 1) * 8 * 4);
    }
  } else {
    pl->off_a = off;  // delta [Hq, T]
    off = align256(off + (size_t)Hq * T * 4);
    if (S > 1) {
      pl->off_b = off;
      off = align256(off + (size_t)S * T * Hq * Dqk * 4);
    }
    // dimension-major packed K of the prompt and of the responses (dQ kernel; latent KV: read from
    // the K tiles by transposed LDS reads)
    if (!wide) {
      pl->off_c = off;
      off = align256(off + (size_t)Hkv * Dqk * pl->ppad * 2);
      pl->off_d = off;
      off = align256(off + (size_t)Hkv * Dqk * pl->tpad * 2);
    }
    // packed query rows of every kv head (dK/dV kernels); latent KV: row-major only
    pl->mpad = (T * g + 63) / 64 * 64;
    pl->off_qr = off;
    off = align256(off + (size_t)Hkv * pl->mpad * Dqk * 2);
    pl->off_or = off;
    off = align256(off + (size_t)Hkv * pl->mpad * Dv * 2);
    if (!wide) {
      pl->off_qt = off;
      off = align256(off + (size_t)Hkv * pl->mpad * Dqk * 2);
      pl->off_ot = off;
      off = align256(off + (size_t)Hkv * pl->mpad * Dv * 2);
    }
    pl->off_rs = off;
    off = align256(off + (size_t)Hkv * pl->mpad * (wide ? 8 : 32));
    pl->off_sc = off;  // fp16 operand scales: partial maxima (8 per block), then the scales
    off = align256(off + (size_t)(kScaleBlocks + 1) * 8 * 4);
  }
  pl->ws_bytes = off;
  return true;
}

}  // namespace lsr
