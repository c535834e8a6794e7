// Host-only stand-ins for the three kernel launchers the C-ABI entry points call (api.cpp), for the
// sanitizer build of the argument validation: each records the call and checks that every buffer
// the host side derived from the caller's workspace lies inside it. No device code, no HIP calls.
#include <cstdio>
#include <cstdlib>

#include "../../prefix_shared_branch_amd/csrc/kernels.h"

namespace harness {
int launches = 0;
const char* ws_base = nullptr;
size_t ws_bytes = 0;
}  // namespace harness

namespace {

void in_ws(const void* p, const char* what) {
  if (!p) return;
  const char* c = static_cast<const char*>(p);
  if (c < harness::ws_base || c >= harness::ws_base + harness::ws_bytes) {
    std::fprintf(stderr, "FAIL: %s outside the workspace\n", what);
    std::exit(3);
  }
}

void check_geom(const lsr::AttnGeom& g) {
  for (int i = 0; i < g.n_resp; ++i)
    if (g.tok0[i + 1] < g.tok0[i] || g.ktok0[i + 1] < g.ktok0[i]) {
      std::fprintf(stderr, "FAIL: offsets not monotone\n");
      std::exit(3);
    }
}

}  // namespace

namespace lsr {

hipError_t launch_attn_fwd(FwdArgs& a, int, int, hipStream_t) {
  ++harness::launches;
  check_geom(a.geo);
  in_ws(a.o_part, "o_part");
  in_ws(a.lse_part, "lse_part");
  in_ws(a.vscale_part, "vscale_part");
  return hipSuccess;
}

hipError_t launch_attn_bwd(BwdArgs& a, int, int, hipStream_t) {
  ++harness::launches;
  check_geom(a.geo);
  const void* ws[] = {a.delta, a.dq_part, a.Qr, a.dOr, a.QT, a.dOT, a.rowstat, a.scale_part};
  const char* names[] = {"delta", "dq_part", "Qr", "dOr", "QT", "dOT", "rowstat", "scale_part"};
  for (int i = 0; i < 8; ++i) in_ws(ws[i], names[i]);
  return hipSuccess;
}

hipError_t launch_grpo(const GrpoArgs& a, bool, hipStream_t) {
  ++harness::launches;
  if (a.n < 1 || a.n > kMaxResp || a.T < 1) {
    std::fprintf(stderr, "FAIL: empty or oversized loss batch\n");
    std::exit(3);
  }
  for (int i = 0; i < a.n; ++i)
    if (a.row_end[i] < 1 || a.row_end[i] > a.T || (i > 0 && a.row_end[i] < a.row_end[i - 1])) {
      std::fprintf(stderr, "FAIL: loss batch row ends\n");
      std::exit(3);
    }
  in_ws(a.row_loss, "row_loss");
  return hipSuccess;
}

}  // namespace lsr
