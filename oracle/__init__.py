"""CPU oracle for branch-replay attention and the clipped-GRPO token objective.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or calls this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP path (no kernels, headers, helpers or tables), and
it is written from the definitions on the LongStraw study notes
(dimensionstp.github.io, "LongStraw" summary): the policy objective of §1-1, the
serial replay with gradient accumulation of §2-1 and §3-2 (4), and the gradient
decomposition of §2-2. Everything is computed in float64 on the bf16 input
values upcast exactly.

Modules:
  attn   replay attention forward/backward by the plain definition (exact softmax)
  brute  independent formulations used to pin `attn`: full causal attention on the
         concatenated [prompt; response] sequence, and the tree-masked whole-group batch
  grpo   group advantages, the clipped per-token objective, its gradient w.r.t. logits
  fd     central finite differences

Parity status: every function here is pinned by tests/test_oracle_*.py against
closed forms, brute force, library routines (torch float64 autograd / SDPA,
scipy log_softmax) or finite differences; nothing is "parity unpinned".
"""
from . import attn, brute, fd, grpo  # noqa: F401
