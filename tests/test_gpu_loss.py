"""GPU parity of ls_grpo_token_loss against the fp64 oracle (clipped objective of the LongStraw
study notes §1-1). Inputs are the seeded generators' bf16 logits; old log-probs are the oracle's
own log-probs plus the generator's noise; the kernel is reached only through the C ABI."""
import numpy as np
import pytest

from oracle import grpo
from prefix_shared_branch_amd import inputs
from tests.helpers import dev_bf16, host_f64

pytestmark = pytest.mark.gpu


def _setup(cfg, lengths=None, V=None):
    import torch
    cfg = inputs.replace(cfg, V=V) if V else cfg
    R = inputs.response_lengths(cfg) if lengths is None else np.asarray(lengths, dtype=np.int32)
    G = len(R)
    rewards = inputs.rewards(inputs.replace(cfg, G=G))
    if rewards.min() == rewards.max():       # keep both signs of advantage in play
        rewards[0] = 1.0 - rewards[0]
    logits_bits = [inputs.logits(cfg, i, 0, int(R[i])) for i in range(G)]
    x = np.concatenate([inputs.bf16_bits_to_f64(b) for b in logits_bits])
    y = np.concatenate([inputs.targets(cfg, i, int(R[i])) for i in range(G)])
    old = (grpo.token_logp(x, y) + np.concatenate([inputs.old_logp_noise(cfg, i, int(R[i])) for i in range(G)])
           ).astype(np.float32)
    d = dict(cfg=cfg, R=R, G=G, rewards=rewards, x=x, y=y, old=old,
             logits=dev_bf16(np.concatenate(logits_bits)), targets=torch.from_numpy(y).cuda(),
             old_d=torch.from_numpy(old).cuda())
    return d


def _run(d, first, count):
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    cu = np.concatenate([[0], np.cumsum(d["R"])])
    r0, r1 = cu[first], cu[first + count]
    T = r1 - r0
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    logp = torch.empty(T, dtype=torch.float32, device="cuda")
    clip = torch.empty(T, dtype=torch.uint8, device="cuda")
    dl = L.ls_grpo_token_loss(d["logits"][r0:r1], d["targets"][r0:r1], d["old_d"][r0:r1], d["R"], d["rewards"],
                              d["cfg"].eps, first, count, loss, logp_out=logp, clipped_out=clip)
    torch.cuda.synchronize()
    return float(loss.item()), dl, logp.cpu().numpy(), clip.cpu().numpy().astype(bool)


def _compare(d, first, count, got):
    cu = np.concatenate([[0], np.cumsum(d["R"])])
    r0, r1 = cu[first], cu[first + count]
    x, y, old = d["x"][r0:r1], d["y"][r0:r1], d["old"][r0:r1]
    loss_ref, dl_ref, logp_ref, clip_ref = grpo.grpo_token_loss(x, y, old, d["R"], d["rewards"], d["G"], d["cfg"].eps,
                                                                first, count)
    s_abs = grpo.abs_term_scale(x, y, old, d["R"], d["rewards"], d["G"], d["cfg"].eps, first, count)
    loss, dl, logp, clip = got
    assert abs(loss - loss_ref) <= 1e-3 * s_abs + 1e-12, (loss, loss_ref, s_abs)
    assert np.max(np.abs(logp - logp_ref)) <= 1e-4
    rho = np.exp(logp_ref - old)
    eps = d["cfg"].eps
    near = (np.abs(rho - (1 + eps)) < 1e-5) | (np.abs(rho - (1 - eps)) < 1e-5)
    assert np.array_equal(clip[~near], clip_ref[~near])
    dlh = host_f64(dl)
    for t in range(r1 - r0):
        if near[t]:
            continue
        if clip_ref[t]:
            assert np.all(dlh[t] == 0.0), f"clipped row {t} not exactly zero"
        else:
            nr = np.linalg.norm(dl_ref[t])
            if nr == 0:
                assert np.all(dlh[t] == 0.0)
            else:
                assert np.linalg.norm(dlh[t] - dl_ref[t]) <= 1e-2 * nr, t
    return clip_ref


@pytest.mark.parametrize("cfgname", ["tiny", "tiny_clip"])
def test_loss_tiny_per_response_and_whole_group(cfgname):
    d = _setup(inputs.CONFIGS[cfgname])
    nclip = 0
    for i in range(d["G"]):
        nclip += _compare(d, i, 1, _run(d, i, 1)).sum()
    _compare(d, 0, d["G"], _run(d, 0, d["G"]))
    if cfgname == "tiny_clip":
        assert nclip > 0


def test_loss_micro_vocab_elementwise_path():
    d = _setup(inputs.CONFIGS["micro"], lengths=[3, 5, 4])
    _compare(d, 0, 3, _run(d, 0, 3))
    _compare(d, 1, 2, _run(d, 1, 2))


def test_loss_full_vocab_151936():
    d = _setup(inputs.CONFIGS["mid"], lengths=[5, 9, 3])
    _compare(d, 0, 3, _run(d, 0, 3))


def test_loss_odd_vocab_aligned_and_ragged():
    d = _setup(inputs.CONFIGS["tiny_clip"], lengths=[4, 6], V=1000)      # V % 8 == 0, not a chunk multiple
    _compare(d, 0, 2, _run(d, 0, 2))
    d = _setup(inputs.CONFIGS["tiny_clip"], lengths=[4, 6], V=1001)      # element-wise path
    _compare(d, 0, 2, _run(d, 0, 2))


def test_loss_equal_rewards_zero_gradient_and_determinism():
    import torch
    d = _setup(inputs.CONFIGS["tiny"], lengths=[7, 9])
    d["rewards"] = np.array([1.0, 1.0], dtype=np.float32)
    loss, dl, _, _ = _run(d, 0, 2)
    assert loss == 0.0 and torch.all(dl == 0).item()
    d = _setup(inputs.CONFIGS["tiny_clip"])
    a = _run(d, 0, d["G"])
    b = _run(d, 0, d["G"])
    assert a[0] == b[0] and torch.equal(a[1], b[1])


def test_loss_invalid_target_gives_nan_row_only():
    import torch
    d = _setup(inputs.CONFIGS["tiny"], lengths=[5])
    d["targets"][2] = 999999
    loss, dl, logp, _ = _run(d, 0, 1)
    assert np.isnan(loss) and np.isnan(logp[2]) and torch.isnan(dl[2].float()).all().item()
    assert np.all(np.isfinite(np.delete(logp, 2)))
    assert torch.isfinite(dl[[0, 1, 3, 4]].float()).all().item()


def _run_scoring(d, first, count):
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    cu = np.concatenate([[0], np.cumsum(d["R"])])
    r0, r1 = cu[first], cu[first + count]
    T = r1 - r0
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    logp = torch.empty(T, dtype=torch.float32, device="cuda")
    clip = torch.empty(T, dtype=torch.uint8, device="cuda")
    dl = L.ls_grpo_token_loss(d["logits"][r0:r1], d["targets"][r0:r1], d["old_d"][r0:r1], d["R"], d["rewards"],
                              d["cfg"].eps, first, count, loss, logp_out=logp, clipped_out=clip, scoring_only=True)
    torch.cuda.synchronize()
    assert dl is None
    return float(loss.item()), logp.cpu().numpy(), clip.cpu().numpy().astype(bool)


@pytest.mark.parametrize("cfgname,lengths,V", [("tiny_clip", None, None), ("mid", [5, 9, 3], None),
                                               ("tiny_clip", [4, 6], 1001)])
def test_loss_scoring_only_matches_full_pass_and_oracle(cfgname, lengths, V):
    """Scoring without dlogits (an old or reference policy pass): same loss, log-probs and clip flags,
    bit for bit, as the pass that writes dlogits, and the oracle's log-probs."""
    d = _setup(inputs.CONFIGS[cfgname], lengths=lengths, V=V)
    G = d["G"]
    loss_f, _, logp_f, clip_f = _run(d, 0, G)
    loss_s, logp_s, clip_s = _run_scoring(d, 0, G)
    assert loss_s == loss_f
    assert np.array_equal(logp_s, logp_f) and np.array_equal(clip_s, clip_f)
    logp_ref = grpo.token_logp(d["x"], d["y"])
    assert np.max(np.abs(logp_s - logp_ref)) <= 1e-4


@pytest.mark.parametrize("cfgname,lengths", [("mid", [170, 120]), ("tiny_clip", [700, 500])])
def test_loss_rows_looped_per_workgroup(cfgname, lengths):
    """More rows than the row loop has workgroups (256 at the full vocabulary, 1024 below it), so a
    workgroup streams several rows, reloading each chunk's registers with the next row's chunk as its
    dlogits are written. Full pass and scoring pass against the oracle; per-response calls (each
    starting the loop afresh) give the same dlogits and log-probs bit for bit."""
    import torch
    d = _setup(inputs.CONFIGS[cfgname], lengths=lengths)
    G = d["G"]
    got = _run(d, 0, G)
    _compare(d, 0, G, got)
    _, logp_s, clip_s = _run_scoring(d, 0, G)
    assert np.array_equal(logp_s, got[2]) and np.array_equal(clip_s, got[3])
    cu = np.concatenate([[0], np.cumsum(d["R"])])
    for i in range(G):
        _, dl_i, logp_i, _ = _run(d, i, 1)
        assert torch.equal(dl_i, got[1][cu[i]:cu[i + 1]])
        assert np.array_equal(logp_i, got[2][cu[i]:cu[i + 1]])


@pytest.mark.parametrize("V", [262144, 262152, 196616])
def test_loss_rows_longer_than_registers(V):
    """Vocabularies above 196,608: the row is streamed twice (running max and rescaled sum, then
    dlogits). Full pass and scoring pass against the oracle."""
    d = _setup(inputs.CONFIGS["tiny_clip"], lengths=[3, 5], V=V)
    got = _run(d, 0, 2)
    _compare(d, 0, 2, got)
    _, logp_s, clip_s = _run_scoring(d, 0, 2)
    assert np.array_equal(logp_s, got[2]) and np.array_equal(clip_s, got[3])
