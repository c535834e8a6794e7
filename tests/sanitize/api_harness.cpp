// Drives the C-ABI entry points of api.cpp on the host, with the kernel launchers replaced by the
// stand-ins of launch_stubs.cpp: every invalid call must return its documented status and launch
// nothing, every valid one LS_OK with the launches it makes. Built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitize.py), so an out-of-bounds read of a host
// array (cu_seqlens, R, rewards), an overflowing size computation or any other undefined behaviour
// in the validation fails the run. Device pointers are aligned addresses into a host block that
// nothing dereferences.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/ls_replay.h"

namespace harness {
extern int launches;
extern const char* ws_base;
extern size_t ws_bytes;
}  // namespace harness

namespace {

int failures = 0;
int checks = 0;

void expect(int line, const char* what, int status, int want, int launched, int want_launches) {
  ++checks;
  if (status != want || launched != want_launches) {
    std::fprintf(stderr, "FAIL line %d: %s -> status %d (want %d), launches %d (want %d)\n", line, what, status, want,
                 launched, want_launches);
    ++failures;
  }
}

#define EXPECT(call, want, want_launches)                                          \
  do {                                                                             \
    const int before_ = harness::launches;                                         \
    const int st_ = (call);                                                        \
    expect(__LINE__, #call, st_, (want), harness::launches - before_, (want_launches)); \
  } while (0)

// host memory standing in for device buffers and workspaces
char* block = nullptr;
constexpr size_t kBlock = 64u << 20;
char* dev(size_t off) { return block + off; }

// a workspace of exactly `bytes` at a 256-byte aligned place in the block
char* workspace(size_t bytes) {
  harness::ws_base = dev(32u << 20);
  harness::ws_bytes = bytes;
  return dev(32u << 20);
}

ls_attn_desc desc(int P, int Hq, int Hkv, int D, int Dv) {
  ls_attn_desc d;
  d.P = P;
  d.Hq = Hq;
  d.Hkv = Hkv;
  d.Dqk = D;
  d.Dv = Dv;
  d.ldk = (int64_t)Hkv * D;
  d.ldv = (int64_t)Hkv * Dv;
  d.softmax_scale = 1.0f / std::sqrt((float)D);
  return d;
}

int fwd(const ls_attn_desc& d, int n, const int32_t* cu, char* ws, size_t wsb, size_t qoff = 0) {
  const void* kp = d.P > 0 ? dev(0) : nullptr;
  const void* vp = d.Dqk == 576 ? kp : (d.P > 0 ? dev(1u << 20) : nullptr);
  const void* ks = dev(2u << 20);
  const void* vs = d.Dqk == 576 ? ks : dev(3u << 20);
  return ls_replay_attn_fwd(nullptr, &d, kp, vp, n, cu, dev((4u << 20) + qoff), ks, vs, dev(5u << 20),
                            reinterpret_cast<float*>(dev(6u << 20)), dev(7u << 20), ws, wsb);
}

int bwd(const ls_attn_desc& d, int n, const int32_t* cu, bool exact, char* ws, size_t wsb, size_t accoff = 0,
        bool one_accum = false) {
  const void* kp = d.P > 0 ? dev(0) : nullptr;
  const void* vp = d.Dqk == 576 ? kp : (d.P > 0 ? dev(1u << 20) : nullptr);
  const void* ks = dev(2u << 20);
  const void* vs = d.Dqk == 576 ? ks : dev(3u << 20);
  float* dkp = exact ? reinterpret_cast<float*>(dev((16u << 20) + accoff)) : nullptr;
  float* dvp = exact && !one_accum ? reinterpret_cast<float*>(dev(17u << 20)) : nullptr;
  return ls_replay_attn_bwd(nullptr, &d, kp, vp, n, cu, dev(4u << 20), ks, vs, dev(5u << 20),
                            reinterpret_cast<float*>(dev(6u << 20)), nullptr, dev(8u << 20), dev(9u << 20),
                            dev(10u << 20), dev(11u << 20), dkp, dvp, ws, wsb);
}

size_t attn_ws(const ls_attn_desc& d, int n, const int32_t* cu, int which) {
  size_t b = 0;
  const int st = ls_replay_attn_workspace_bytes(&d, n, cu, which, &b);
  if (st != LS_OK) {
    std::fprintf(stderr, "FAIL: workspace query %d\n", st);
    ++failures;
  }
  return b;
}

void attention() {
  const int32_t cu[3] = {0, 37, 100};
  for (int D : {64, 128}) {
    ls_attn_desc d = desc(1000, 8, 2, D, D);
    const size_t wf = attn_ws(d, 2, cu, 0), wb = attn_ws(d, 2, cu, 1), wr = attn_ws(d, 2, cu, 2);
    EXPECT(fwd(d, 2, cu, workspace(wf), wf), LS_OK, 1);
    EXPECT(bwd(d, 2, cu, true, workspace(wb), wb), LS_OK, 1);
    EXPECT(bwd(d, 2, cu, false, workspace(wr), wr), LS_OK, 1);
    if (wf > 0) EXPECT(fwd(d, 2, cu, workspace(wf), wf - 1), LS_ERR_WORKSPACE, 0);
    if (wb > 0) EXPECT(bwd(d, 2, cu, true, workspace(wb), wb - 1), LS_ERR_WORKSPACE, 0);
    if (wf > 0) EXPECT(fwd(d, 2, cu, nullptr, wf), LS_ERR_WORKSPACE, 0);
    if (wf > 0) EXPECT(fwd(d, 2, cu, workspace(wf + 64) + 64, wf), LS_ERR_WORKSPACE, 0);   // misaligned
    EXPECT(fwd(d, 2, cu, workspace(wf), wf, 8), LS_ERR_INVALID_ARG, 0);                      // misaligned Q
    EXPECT(bwd(d, 2, cu, true, workspace(wb), wb, 4), LS_ERR_INVALID_ARG, 0);                // misaligned dKp
    EXPECT(bwd(d, 2, cu, true, workspace(wb), wb, 0, true), LS_ERR_INVALID_ARG, 0);          // one accumulator
  }
  ls_attn_desc d = desc(1000, 8, 2, 64, 64);
  const size_t big = 16u << 20;
  const int32_t empty[2] = {0, 0};
  EXPECT(fwd(d, 1, empty, workspace(big), big), LS_OK, 0);                                   // T == 0
  ls_attn_desc e = d;
  e.Hq = 6;
  e.Hkv = 4;
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);                         // Hq % Hkv
  e = desc(1000, 8, 2, 96, 96);
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_UNSUPPORTED, 0);                         // head dim
  e = desc(1000, 8, 2, 64, 128);
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);                         // Dv > Dqk
  e = d;
  e.softmax_scale = NAN;
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);
  e.softmax_scale = 0.0f;
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);
  e = d;
  e.ldk = 64;
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);                         // ldk < Hkv Dqk
  e.ldk = 132;
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);                         // ldk % 8
  e = d;
  e.P = -1;
  EXPECT(fwd(e, 2, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);
  EXPECT(fwd(d, 0, cu, workspace(big), big), LS_ERR_INVALID_ARG, 0);                         // n_resp 0
  std::vector<int32_t> many(LS_MAX_RESPONSES_PER_CALL + 2);
  for (size_t i = 0; i < many.size(); ++i) many[i] = (int32_t)i;
  EXPECT(fwd(d, LS_MAX_RESPONSES_PER_CALL + 1, many.data(), workspace(big), big), LS_ERR_UNSUPPORTED, 0);
  const size_t wm = attn_ws(d, LS_MAX_RESPONSES_PER_CALL, many.data(), 0);
  EXPECT(fwd(d, LS_MAX_RESPONSES_PER_CALL, many.data(), workspace(wm), wm), LS_OK, 1);
  const int32_t bad0[3] = {1, 37, 100}, down[3] = {0, 37, 20};
  EXPECT(fwd(d, 2, bad0, workspace(big), big), LS_ERR_INVALID_ARG, 0);
  EXPECT(fwd(d, 2, down, workspace(big), big), LS_ERR_INVALID_ARG, 0);
  const int32_t huge[2] = {0, 0x7fffff00};
  EXPECT(fwd(d, 1, huge, workspace(big), big), LS_ERR_UNSUPPORTED, 0);                       // 32-bit sizes
  EXPECT(ls_replay_attn_fwd(nullptr, &d, dev(0), dev(1u << 20), 2, cu, dev(4u << 20), dev(2u << 20),
                            dev(3u << 20), nullptr, reinterpret_cast<float*>(dev(6u << 20)), nullptr,
                            workspace(big), big),
         LS_ERR_INVALID_ARG, 0);                                                             // O missing
  EXPECT(ls_replay_attn_fwd(nullptr, nullptr, dev(0), dev(1u << 20), 2, cu, dev(4u << 20), dev(2u << 20),
                            dev(3u << 20), dev(5u << 20), reinterpret_cast<float*>(dev(6u << 20)), nullptr,
                            workspace(big), big),
         LS_ERR_INVALID_ARG, 0);                                                             // no desc
  size_t b = 0;
  EXPECT(ls_replay_attn_workspace_bytes(&d, 2, cu, 3, &b), LS_ERR_INVALID_ARG, 0);
  EXPECT(ls_replay_attn_workspace_bytes(&d, 2, cu, 0, nullptr), LS_ERR_INVALID_ARG, 0);

  // no prompt: K/V pointers may be null
  ls_attn_desc np = desc(0, 8, 2, 128, 128);
  const size_t w0 = attn_ws(np, 2, cu, 1);
  EXPECT(bwd(np, 2, cu, true, workspace(w0), w0), LS_OK, 1);

  // latent KV: one kv head, V aliasing K
  ls_attn_desc w = desc(300, 4, 1, 576, 512);
  w.ldv = w.ldk;
  const size_t ww = attn_ws(w, 2, cu, 0), wwb = attn_ws(w, 2, cu, 1);
  EXPECT(fwd(w, 2, cu, workspace(ww), ww), LS_OK, 1);
  EXPECT(bwd(w, 2, cu, true, workspace(wwb), wwb), LS_OK, 1);
  EXPECT(ls_replay_attn_fwd(nullptr, &w, dev(0), dev(1u << 20), 2, cu, dev(4u << 20), dev(2u << 20), dev(2u << 20),
                            dev(5u << 20), reinterpret_cast<float*>(dev(6u << 20)), nullptr, workspace(ww), ww),
         LS_ERR_UNSUPPORTED, 0);                                                             // V not aliasing K
  ls_attn_desc w2 = w;
  w2.Hq = 4;
  w2.Hkv = 2;
  w2.ldk = w2.ldv = 2 * 576;
  EXPECT(fwd(w2, 2, cu, workspace(big), big), LS_ERR_UNSUPPORTED, 0);                        // two kv heads
}

void blocks() {
  ls_attn_desc d = desc(500, 8, 2, 128, 128);
  size_t wf = 0, wb = 0;
  EXPECT(ls_replay_attn_block_workspace_bytes(&d, 40, 24, 0, &wf), LS_OK, 0);
  EXPECT(ls_replay_attn_block_workspace_bytes(&d, 40, 24, 1, &wb), LS_OK, 0);
  EXPECT(ls_replay_attn_block_workspace_bytes(&d, -1, 24, 0, &wf), LS_ERR_INVALID_ARG, 0);
  float* acc = reinterpret_cast<float*>(dev(12u << 20));
  EXPECT(ls_replay_attn_fwd_block(nullptr, &d, dev(0), dev(1u << 20), 40, 24, dev(4u << 20), dev(2u << 20),
                                  dev(3u << 20), dev(5u << 20), reinterpret_cast<float*>(dev(6u << 20)), nullptr,
                                  workspace(wf), wf),
         LS_OK, 1);
  EXPECT(ls_replay_attn_fwd_block(nullptr, &d, dev(0), dev(1u << 20), 40, 0, dev(4u << 20), dev(2u << 20),
                                  dev(3u << 20), dev(5u << 20), reinterpret_cast<float*>(dev(6u << 20)), nullptr,
                                  workspace(wf), wf),
         LS_OK, 0);                                                                          // nq == 0
  EXPECT(ls_replay_attn_fwd_block(nullptr, &d, dev(0), dev(1u << 20), 0x7ffffff0, 0x100, dev(4u << 20),
                                  dev(2u << 20), dev(3u << 20), dev(5u << 20), reinterpret_cast<float*>(dev(6u << 20)),
                                  nullptr, workspace(wf), wf),
         LS_ERR_INVALID_ARG, 0);                                                             // q0 + nq overflows
  EXPECT(ls_replay_attn_bwd_block(nullptr, &d, dev(0), dev(1u << 20), 40, 24, dev(4u << 20), dev(2u << 20),
                                  dev(3u << 20), dev(5u << 20), reinterpret_cast<float*>(dev(6u << 20)), nullptr,
                                  dev(8u << 20), dev(9u << 20), acc, acc + 65536,
                                  reinterpret_cast<float*>(dev(16u << 20)), reinterpret_cast<float*>(dev(17u << 20)),
                                  workspace(wb), wb),
         LS_OK, 1);
  EXPECT(ls_replay_attn_bwd_block(nullptr, &d, dev(0), dev(1u << 20), 40, 24, dev(4u << 20), dev(2u << 20),
                                  dev(3u << 20), dev(5u << 20), reinterpret_cast<float*>(dev(6u << 20)), nullptr,
                                  dev(8u << 20), dev(9u << 20), nullptr, acc + 65536,
                                  reinterpret_cast<float*>(dev(16u << 20)), reinterpret_cast<float*>(dev(17u << 20)),
                                  workspace(wb), wb),
         LS_ERR_INVALID_ARG, 0);                                                             // accumulator missing
}

int loss(int V, int G, const int32_t* R, const float* rw, float eps, int first, int count, size_t wsb,
         void* logits = nullptr) {
  return ls_grpo_token_loss(nullptr, V, G, R, rw, eps, first, count, logits ? logits : dev(0),
                            reinterpret_cast<const int32_t*>(dev(20u << 20)),
                            reinterpret_cast<const float*>(dev(21u << 20)), dev(22u << 20),
                            reinterpret_cast<float*>(dev(23u << 20)), reinterpret_cast<float*>(dev(24u << 20)),
                            reinterpret_cast<uint8_t*>(dev(25u << 20)), workspace(wsb), wsb);
}

void grpo() {
  const int32_t R[3] = {5, 7, 9};
  const float rw[3] = {1.0f, 0.0f, 0.5f};
  size_t w = 0;
  EXPECT(ls_grpo_workspace_bytes(21, 4096, &w), LS_OK, 0);
  EXPECT(ls_grpo_workspace_bytes(-1, 4096, &w), LS_ERR_INVALID_ARG, 0);
  EXPECT(loss(4096, 3, R, rw, 0.2f, 0, 3, w), LS_OK, 1);
  EXPECT(loss(4096, 3, R, rw, 0.2f, 1, 1, w), LS_OK, 1);
  EXPECT(loss(4096, 3, R, rw, 0.2f, 0, 3, w - 1), LS_ERR_WORKSPACE, 0);
  EXPECT(loss(0, 3, R, rw, 0.2f, 0, 3, w), LS_ERR_INVALID_ARG, 0);
  EXPECT(loss((1 << 24) + 8, 3, R, rw, 0.2f, 0, 3, w), LS_ERR_UNSUPPORTED, 0);
  EXPECT(loss(4096, 3, R, rw, 0.0f, 0, 3, w), LS_ERR_INVALID_ARG, 0);
  EXPECT(loss(4096, 3, R, rw, 1.0f, 0, 3, w), LS_ERR_INVALID_ARG, 0);
  EXPECT(loss(4096, 3, R, rw, NAN, 0, 3, w), LS_ERR_INVALID_ARG, 0);
  EXPECT(loss(4096, 3, R, rw, 0.2f, 2, 2, w), LS_ERR_INVALID_ARG, 0);                        // past G
  EXPECT(loss(4096, 3, R, rw, 0.2f, -1, 1, w), LS_ERR_INVALID_ARG, 0);
  const int32_t R0[3] = {5, 0, 9};
  EXPECT(loss(4096, 3, R0, rw, 0.2f, 0, 3, w), LS_ERR_INVALID_ARG, 0);                       // empty response
  const float rnan[3] = {1.0f, NAN, 0.5f};
  EXPECT(loss(4096, 3, R, rnan, 0.2f, 0, 3, w), LS_ERR_INVALID_ARG, 0);
  EXPECT(loss(4096, 3, R, rw, 0.2f, 0, 3, w, dev(22u << 20)), LS_ERR_INVALID_ARG, 0);        // dlogits aliases
  // 70 responses: two launches of at most 64 responses each
  std::vector<int32_t> R70(70, 2);
  std::vector<float> r70(70);
  for (int i = 0; i < 70; ++i) r70[i] = (float)(i % 3);
  size_t w70 = 0;
  EXPECT(ls_grpo_workspace_bytes(140, 4096, &w70), LS_OK, 0);
  EXPECT(loss(4096, 70, R70.data(), r70.data(), 0.2f, 0, 70, w70), LS_OK, 2);
  const int32_t big[2] = {0x7fff0000, 0x7fff0000};
  const float rb[2] = {0.0f, 1.0f};
  EXPECT(loss(8, 2, big, rb, 0.2f, 0, 2, 1u << 20), LS_ERR_UNSUPPORTED, 0);                  // T > 2^31 - 1
}

}  // namespace

int main() {
  block = static_cast<char*>(std::aligned_alloc(4096, kBlock));
  attention();
  blocks();
  grpo();
  std::free(block);
  std::printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
