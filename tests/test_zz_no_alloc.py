"""The loss entry point that allocates nothing (ls_grpo_token_loss_noalloc) against the workspace
entry point (ls_grpo_token_loss) through the C ABI.

Both run the same kernels on the same rows, so every output must match bit for bit: the loss share,
dlogits, log-probs and clip flags of the clipped-GRPO objective (LongStraw study notes §1-1,
L_policy). Two calls in a row, the second over fewer rows than the first, show that the fixed
scratch array keeps no state the next call depends on; a call over more rows than the array holds is
refused before anything runs."""
import numpy as np
import pytest

from oracle import grpo
from prefix_shared_branch_amd import inputs
from tests.helpers import dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(cfg, lengths):
    import torch
    R = np.asarray(lengths, dtype=np.int32)
    T = int(R.sum())
    x_bits = np.concatenate([inputs.logits(cfg, i, 0, int(R[i])) for i in range(len(R))])
    y = np.concatenate([inputs.targets(cfg, i, int(R[i])) for i in range(len(R))])
    x = inputs.bf16_bits_to_f64(x_bits)
    old = np.concatenate([grpo.token_logp(x[int(a):int(b)], y[int(a):int(b)]) + inputs.old_logp_noise(cfg, i, int(R[i]))
                          for i, (a, b) in enumerate(zip(np.r_[0, np.cumsum(R)[:-1]], np.cumsum(R)))])
    return R, T, dev_bf16(x_bits), torch.from_numpy(y.astype(np.int32)).cuda(), \
        torch.from_numpy(old.astype(np.float32)).cuda()


def _both(cfg, R, T, logits, y, old, first, count, rows):
    """One call of each entry point over responses [first, first+count) (their rows packed)."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    rewards = inputs.rewards(cfg)[:len(R)]
    sl = slice(rows[0], rows[1])
    out = []
    for noalloc in (False, True):
        loss = torch.zeros(1, dtype=torch.float32, device="cuda")
        dl = torch.empty(rows[1] - rows[0], cfg.V, dtype=torch.bfloat16, device="cuda")
        lp = torch.empty(rows[1] - rows[0], dtype=torch.float32, device="cuda")
        cl = torch.empty(rows[1] - rows[0], dtype=torch.uint8, device="cuda")
        if noalloc:
            L.ls_grpo_token_loss_noalloc(logits[sl], y[sl], old[sl], R, rewards, cfg.eps, first, count, loss, dl,
                                         logp_out=lp, clipped_out=cl)
        else:
            L.ls_grpo_token_loss(logits[sl], y[sl], old[sl], R, rewards, cfg.eps, first, count, loss, dlogits=dl,
                                 logp_out=lp, clipped_out=cl)
        torch.cuda.synchronize()
        out.append((loss, dl, lp, cl))
    return out


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    cfg = inputs.replace(inputs.CONFIGS["mid"], seed=61)
    R, T, logits, y, old = _inputs(cfg, [300, 220, 190])
    cuts = np.r_[0, np.cumsum(R)]
    # first call: all three responses; second call: the last response alone (fewer rows)
    for first, count in ((0, 3), (2, 1)):
        rows = (int(cuts[first]), int(cuts[first + count]))
        print(f"[noalloc] V={cfg.V} responses {first}..{first + count - 1}, rows {rows}", flush=True)
        (l0, d0, p0, c0), (l1, d1, p1, c1) = _both(cfg, R, T, logits, y, old, first, count, rows)
        assert torch.equal(l0, l1), (float(l0), float(l1))
        assert torch.equal(d0.view(torch.int16), d1.view(torch.int16))
        assert torch.equal(p0, p1)
        assert torch.equal(c0, c1)


def test_noalloc_refuses_more_rows_than_its_array():
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    n = L.LS_NOALLOC_MAX_ROWS + 1
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    buf = torch.empty(64, dtype=torch.int32, device="cuda")   # never read: the row count is refused first
    Ra, Rp = L._i32_array([n])
    ra, rp = L._f32_array([1.0])
    p = buf.data_ptr()
    code = L.lib().ls_grpo_token_loss_noalloc(L._stream(), 8, 1, Rp, rp, 0.2, 0, 1, p, p, p, None, loss.data_ptr(),
                                              None, None)
    assert code == L.LS_ERR_WORKSPACE, L.ls_status_string(code)
