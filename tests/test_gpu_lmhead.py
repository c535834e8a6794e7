"""GPU parity of ls_grpo_lmhead_loss (LM head, logits = H W^T chunk by chunk, fused with the clipped
GRPO objective of the LongStraw study notes §1-1) against the fp64 oracle in oracle/lmhead.py.

The oracle rounds the logits to bf16 as the device does (one fp32 accumulation, then bf16). Its
fp64 product and the device's fp32 one can round to neighbouring bf16 values where the product sits
next to a rounding midpoint; tokens whose target logit is such a case, or whose ratio sits at a clip
boundary, are compared with one bf16 step of slack (log-probs) or not at all (clip flags)."""
import numpy as np
import pytest

from oracle import grpo, lmhead
from prefix_shared_branch_amd import inputs
from tests.helpers import check_bf16_out, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


def _setup(cfg, lengths, d):
    import torch
    R = np.asarray(lengths, dtype=np.int32)
    G = len(R)
    rewards = inputs.rewards(inputs.replace(cfg, G=G))
    if rewards.min() == rewards.max():
        rewards[0] = 1.0 - rewards[0]
    hb = np.concatenate([inputs.hidden(cfg, i, 0, int(R[i]), d) for i in range(G)])
    wb = inputs.projection(cfg, d)
    Hf, Wf = inputs.bf16_bits_to_f64(hb), inputs.bf16_bits_to_f64(wb)
    y = np.concatenate([inputs.targets(cfg, i, int(R[i])) for i in range(G)])
    x64 = Hf @ Wf.T
    old = (grpo.token_logp(lmhead.round_bf16(x64), y)
           + np.concatenate([inputs.old_logp_noise(cfg, i, int(R[i])) for i in range(G)])).astype(np.float32)
    return dict(R=R, G=G, rewards=rewards, Hf=Hf, Wf=Wf, y=y, old=old, x64=x64, H=dev_bf16(hb), W=dev_bf16(wb),
                targets=torch.from_numpy(y).cuda(), old_d=torch.from_numpy(old).cuda(), eps=cfg.eps, V=cfg.V, d=d)


def _run(s, scoring_only=False, first=0, count=None):
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    count = s["G"] - first if count is None else count
    T = int(s["R"][first:first + count].sum())
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    logp = torch.empty(T, dtype=torch.float32, device="cuda")
    clip = torch.empty(T, dtype=torch.uint8, device="cuda")
    dW = None if scoring_only else torch.zeros(s["V"], s["d"], dtype=torch.float32, device="cuda")
    cu = np.concatenate([[0], np.cumsum(s["R"])])
    r0, r1 = int(cu[first]), int(cu[first + count])
    dH = L.ls_grpo_lmhead_loss(s["H"][r0:r1], s["W"], s["targets"][r0:r1], s["old_d"][r0:r1], s["R"], s["rewards"],
                               s["eps"], first, count, loss, dW_accum=dW, logp_out=logp, clipped_out=clip,
                               scoring_only=scoring_only)
    torch.cuda.synchronize()
    return loss, dH, dW, logp, clip


def _ambiguous(x64):
    """Products whose fp64 and fp32 forms may round to different bf16 neighbours."""
    return lmhead.round_bf16(x64 * (1 + 2.0 ** -20)) != lmhead.round_bf16(x64 * (1 - 2.0 ** -20))


def _check(s, got, first=0, count=None):
    loss, dH, dW, logp, clip = got
    G, R, eps = s["G"], s["R"], s["eps"]
    count = G - first if count is None else count
    cu = np.concatenate([[0], np.cumsum(R)])
    sl = slice(int(cu[first]), int(cu[first + count]))
    y, old, x64 = s["y"][sl], s["old"][sl], s["x64"][sl]
    l_ref, dH_ref, dW_ref, logp_ref, clip_ref = lmhead.lmhead_grpo_loss(s["Hf"][sl], s["Wf"], y, old, R,
                                                                        s["rewards"], G, eps, first, count)
    x = lmhead.round_bf16(x64)
    S_abs = grpo.abs_term_scale(x, y, old, R, s["rewards"], G, eps, first, count)
    assert abs(float(loss.item()) - l_ref) <= 1e-3 * S_abs, (float(loss.item()), l_ref, S_abs)
    T = len(y)
    xt = x64[np.arange(T), y]
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(xt), 1e-30))) - 7)   # one bf16 step at the target logit
    slack = np.where(_ambiguous(xt), step, 0.0)
    dl = np.abs(host_f64(logp) - logp_ref)
    assert np.all(dl <= 1e-4 + slack), np.max(dl - slack)
    rho = np.exp(logp_ref - old.astype(np.float64))
    sure = (np.abs(rho - (1 - eps)) > 1e-3) & (np.abs(rho - (1 + eps)) > 1e-3)
    np.testing.assert_array_equal(host_f64(clip)[sure].astype(bool), clip_ref[sure])
    if dH is not None:
        check_bf16_out(host_f64(dH)[:, None, :], dH_ref[:, None, :], "dH", literal_abs=False)
        check_bf16_out(host_f64(dW)[:, None, :], dW_ref[:, None, :], "dW", literal_abs=False)
    return l_ref


@pytest.mark.parametrize("cfg_name,lengths,d", [
    ("tiny", [70, 1500, 900], 256),       # 2,470 tokens: two chunks, a response across the boundary
    ("tiny_clip", [33, 64], 96),          # clipped tokens in play
    ("mid", [40, 60], 64),                # the full 151,936-word vocabulary
    ("mid", [9, 14], 32),                 # V = 262,144 below: rows read twice by the streaming kernel
])
def test_lmhead_loss_matches_oracle(cfg_name, lengths, d):
    cfg = inputs.CONFIGS[cfg_name]
    if d == 32:
        cfg = inputs.replace(cfg, V=262144)
    s = _setup(cfg, lengths, d)
    _check(s, _run(s))


def test_lmhead_middle_response_of_a_group():
    """A call over response 1 only: the advantages still come from all G rewards."""
    s = _setup(inputs.CONFIGS["tiny"], [50, 2100, 30], 128)
    _check(s, _run(s, first=1, count=1), first=1, count=1)


def test_lmhead_scoring_only_and_accumulation():
    """Scoring mode gives the same loss share and log-probs with no gradient work; a second call adds
    its dW into the same accumulator."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    s = _setup(inputs.CONFIGS["tiny"], [300, 200], 128)
    loss, dH, dW, logp, clip = _run(s)
    loss2, _, _, logp2, clip2 = _run(s, scoring_only=True)
    assert torch.equal(loss, loss2) and torch.equal(logp, logp2) and torch.equal(clip, clip2)
    loss3 = torch.zeros(1, dtype=torch.float32, device="cuda")
    L.ls_grpo_lmhead_loss(s["H"], s["W"], s["targets"], s["old_d"], s["R"], s["rewards"], s["eps"], 0, s["G"],
                          loss3, dW_accum=dW)
    torch.cuda.synchronize()
    _, _, dW1, _, _ = _run(s)
    assert torch.allclose(dW, 2 * dW1, rtol=1e-6, atol=0)   # the same sums added twice


def test_lmhead_ragged_shapes():
    """Hidden size 40 (a k tail of 8 in the logits product), V = 1,000 (a partial 128-word slab and a
    partial vocabulary tile), token counts that fill no tile."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], V=1000)
    s = _setup(cfg, [70, 131], 40)
    _check(s, _run(s))


def test_lmhead_many_short_responses():
    """70 responses of 1-3 tokens in one chunk: the row kernel runs in batches of at most 64 responses."""
    R = [1 + (i % 3) for i in range(70)]
    s = _setup(inputs.CONFIGS["tiny"], R, 64)
    _check(s, _run(s))


def test_lmhead_two_chunks():
    """4,500 tokens: two chunks of the call, a response across their boundary, and a shorter last chunk
    (its dH product split differently)."""
    s = _setup(inputs.CONFIGS["tiny"], [3000, 1500], 64)
    _check(s, _run(s))


def test_lmhead_full_shape_sampled_rows():
    """The benchmark's shape: one response of 4,096 tokens, d = 5,120, V = 151,936, in the launch
    configuration the benchmark times. The oracle forms the logits of a few sampled tokens (fp64, W
    taken in row blocks) and checks their log-probs, clip flags and dH rows."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    cfg = inputs.CONFIGS["million"]
    R0, d = 4096, cfg.Hq * cfg.Dqk
    R = np.array([R0] + [int(r) for r in inputs.response_lengths(cfg)[1:]], dtype=np.int32)
    G = len(R)
    rewards = inputs.rewards(cfg)
    hb = inputs.hidden(cfg, 0, 0, R0, d)
    y = inputs.targets(cfg, 0, R0)
    rows = np.array([0, 1, 777, 2048, 3001, 4095])
    Hs = inputs.bf16_bits_to_f64(hb[rows])
    blk = 16384
    x = np.zeros((len(rows), cfg.V))
    for v0 in range(0, cfg.V, blk):
        Wb = inputs.bf16_bits_to_f64(inputs.normal_bf16_rows(cfg.seed, inputs.TID_PROJ, 0, v0, min(cfg.V, v0 + blk), d,
                                                              cfg.logit_sigma / float(np.sqrt(d))))
        x[:, v0:v0 + Wb.shape[0]] = Hs @ Wb.T
    xr = lmhead.round_bf16(x)
    noise = inputs.old_logp_noise(cfg, 0, R0)
    old = np.full(R0, -12.0, dtype=np.float32)
    old[rows] = (grpo.token_logp(xr, y[rows]) + noise[rows]).astype(np.float32)
    # the sampled rows through the oracle: weight 1/(G R0) and advantage A_0 enter only as their
    # product (a positive factor), so each row is a one-token response with A scaled to match
    A0 = grpo.advantages(rewards)[0]
    dl = np.zeros_like(x)
    logp_ref = np.zeros(len(rows))
    clip_ref = np.zeros(len(rows), dtype=bool)
    for k in range(len(rows)):
        _, dlk, lpk, ck = grpo.grpo_token_loss(xr[k:k + 1], y[rows[k:k + 1]], old[rows[k:k + 1]], [1], [0.0], 1,
                                               cfg.eps, 0, 1, A=[A0 / (G * R0)])
        dl[k], logp_ref[k], clip_ref[k] = dlk[0], lpk[0], ck[0]
    dH_ref = np.zeros((len(rows), d))
    for v0 in range(0, cfg.V, blk):
        Wb = inputs.bf16_bits_to_f64(inputs.normal_bf16_rows(cfg.seed, inputs.TID_PROJ, 0, v0, min(cfg.V, v0 + blk), d,
                                                              cfg.logit_sigma / float(np.sqrt(d))))
        dH_ref += dl[:, v0:v0 + Wb.shape[0]] @ Wb
    H = dev_bf16(hb)
    W = dev_bf16(inputs.projection(cfg, d))
    dW = torch.zeros(cfg.V, d, dtype=torch.float32, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    logp = torch.empty(R0, dtype=torch.float32, device="cuda")
    clip = torch.empty(R0, dtype=torch.uint8, device="cuda")
    dH = L.ls_grpo_lmhead_loss(H, W, torch.from_numpy(y).cuda(), torch.from_numpy(old).cuda(), R, rewards, cfg.eps,
                               0, 1, loss, dW_accum=dW, logp_out=logp, clipped_out=clip)
    torch.cuda.synchronize()
    assert torch.isfinite(dW).all() and torch.isfinite(dH.float()).all()
    xt = x[np.arange(len(rows)), y[rows]]
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(xt), 1e-30))) - 7)
    slack = np.where(_ambiguous(xt), step, 0.0)
    got_lp = host_f64(logp)[rows]
    assert np.all(np.abs(got_lp - logp_ref) <= 1e-4 + slack), np.abs(got_lp - logp_ref)
    rho = np.exp(logp_ref - old[rows].astype(np.float64))
    sure = (np.abs(rho - (1 - cfg.eps)) > 1e-3) & (np.abs(rho - (1 + cfg.eps)) > 1e-3)
    np.testing.assert_array_equal(host_f64(clip)[rows].astype(bool)[sure], clip_ref[sure])
    check_bf16_out(host_f64(dH)[rows][:, None, :], dH_ref[:, None, :], "dH rows", literal_abs=False)
