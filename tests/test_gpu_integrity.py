"""Integrity of the C-ABI calls on the GPU.

* Guard bands: every output buffer, accumulator and workspace a call is given sits between two
  4 KB bands of a known byte pattern; after the call the bands must be unchanged (no write lands
  outside the bytes the call owns).
* Checkpoint / resume: the prompt-gradient accumulators and the loss are caller-owned (LongStraw
  study notes §2-1: serial replay adds each response's share into them), so a group can stop at any
  response boundary: copy them to the host, drop every device buffer, restore and continue. The
  result must be bitwise equal to the uninterrupted replay.
"""
import numpy as np
import pytest

from prefix_shared_branch_amd import inputs
from tests.helpers import dev_bf16

pytestmark = pytest.mark.gpu

GUARD = 4096
PAT = 0xA5


class Guarded:
    """Buffers carved out of larger allocations whose surplus bytes hold PAT."""

    def __init__(self):
        import torch
        self.t = torch
        self.bufs = []

    def alloc(self, name, shape, dtype, zero=False):
        t = self.t
        n = int(np.prod(shape)) if len(shape) else 1
        nbytes = n * t.tensor([], dtype=dtype).element_size()
        raw = t.full((GUARD + (nbytes + 255) // 256 * 256 + GUARD,), PAT, dtype=t.uint8, device="cuda")
        mid = raw[GUARD:GUARD + nbytes]
        if zero:
            mid.zero_()
        self.bufs.append((name, raw, nbytes))
        return mid.view(dtype).view(*shape)

    def check(self):
        self.t.cuda.synchronize()
        for name, raw, nbytes in self.bufs:
            head, tail = raw[:GUARD], raw[GUARD + nbytes:]
            assert bool((head == PAT).all()), f"{name}: bytes written before the buffer"
            assert bool((tail == PAT).all()), f"{name}: bytes written after the buffer"


def _attn_inputs(cfg, lengths):
    T = int(sum(lengths))
    kp = dev_bf16(inputs.prompt_k(cfg))
    ks = dev_bf16(inputs.suffix_k(cfg, 0, T))
    if cfg.mla:
        vp, vs = kp[:, :, :cfg.Dv], ks[:, :, :cfg.Dv]
    else:
        vp, vs = dev_bf16(inputs.prompt_v(cfg)), dev_bf16(inputs.suffix_v(cfg, 0, T))
    return kp, vp, dev_bf16(inputs.suffix_q(cfg, 0, T)), ks, vs, dev_bf16(inputs.suffix_do(cfg, 0, T))


@pytest.mark.parametrize("D", [64, 128, 576])
def test_attention_guard_bands(D):
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    if D == 576:
        cfg = inputs.replace(inputs.CONFIGS["mla"], P=700, Hq=4, seed=41)
    else:
        cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=6, Hkv=2, Dqk=D, Dv=D, P=900, seed=41)
    lengths = [45, 130]
    cu = inputs.cu_seqlens(np.asarray(lengths))
    T = int(cu[-1])
    kp, vp, q, ks, vs, do = _attn_inputs(cfg, lengths)
    desc = L.make_desc(q, kp, vp, ks, vs, cfg.scale)
    g = Guarded()
    o = g.alloc("O", (T, cfg.Hq, cfg.Dv), torch.bfloat16)
    lse = g.alloc("LSE", (cfg.Hq, T), torch.float32)
    lo = g.alloc("O_lo", (T, cfg.Hq, cfg.Dv), torch.bfloat16)
    wf = g.alloc("fwd workspace", (L.ls_replay_attn_workspace_bytes(desc, cu, 0),), torch.uint8)
    L.ls_replay_attn_fwd(q, ks, vs, kp, vp, cu, cfg.scale, out=o, lse=lse, workspace=wf, o_lo=lo)
    dq = g.alloc("dQ", (T, cfg.Hq, cfg.Dqk), torch.bfloat16)
    dks = g.alloc("dKs", (T, cfg.Hkv, cfg.Dqk), torch.bfloat16)
    dvs = g.alloc("dVs", (T, cfg.Hkv, cfg.Dv), torch.bfloat16)
    dkp = g.alloc("dKp", (cfg.P, cfg.Hkv, cfg.Dqk), torch.float32, zero=True)
    dvp = g.alloc("dVp", (cfg.P, cfg.Hkv, cfg.Dv), torch.float32, zero=True)
    wb = g.alloc("bwd workspace", (L.ls_replay_attn_workspace_bytes(desc, cu, 1),), torch.uint8)
    L.ls_replay_attn_bwd(q, ks, vs, kp, vp, cu, o, lse, do, dkp, dvp, cfg.scale, dq=dq, dks=dks, dvs=dvs,
                         workspace=wb, o_lo=lo)
    # blockwise replay of the second response's rows 20 .. 99 (its keys 0 .. 99)
    r0 = int(cu[1])
    q0, nq = 20, 80
    qb, ksb, vsb, dob = q[r0 + q0:r0 + q0 + nq], ks[r0:r0 + q0 + nq], vs[r0:r0 + q0 + nq], do[r0 + q0:r0 + q0 + nq]
    bdesc = L.make_desc(qb, kp, vp, ksb, vsb, cfg.scale)
    ob = g.alloc("block O", (nq, cfg.Hq, cfg.Dv), torch.bfloat16)
    lseb = g.alloc("block LSE", (cfg.Hq, nq), torch.float32)
    wbf = g.alloc("block fwd workspace", (L.ls_replay_attn_block_workspace_bytes(bdesc, q0, nq, 0),), torch.uint8)
    L.ls_replay_attn_fwd_block(qb, ksb, vsb, kp, vp, q0, cfg.scale, out=ob, lse=lseb, workspace=wbf)
    dqb = g.alloc("block dQ", (nq, cfg.Hq, cfg.Dqk), torch.bfloat16)
    dksa = g.alloc("block dKs accumulator", (q0 + nq, cfg.Hkv, cfg.Dqk), torch.float32, zero=True)
    dvsa = g.alloc("block dVs accumulator", (q0 + nq, cfg.Hkv, cfg.Dv), torch.float32, zero=True)
    wbb = g.alloc("block bwd workspace", (L.ls_replay_attn_block_workspace_bytes(bdesc, q0, nq, 1),), torch.uint8)
    L.ls_replay_attn_bwd_block(qb, ksb, vsb, kp, vp, q0, ob, lseb, dob, dksa, dvsa, dkp, dvp, cfg.scale, dq=dqb,
                               workspace=wbb)
    g.check()
    assert bool(torch.isfinite(dkp).all()) and bool(torch.isfinite(dq.float()).all())


@pytest.mark.parametrize("V", [4096, 1000, 262144])
def test_loss_guard_bands(V):
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    cfg = inputs.replace(inputs.CONFIGS["tiny"], V=V, seed=42)
    R = np.array([7, 20], dtype=np.int32)
    T = int(R.sum())
    lg = dev_bf16(np.concatenate([inputs.logits(cfg, i, 0, int(R[i])) for i in range(2)]))
    y = torch.from_numpy(np.concatenate([inputs.targets(cfg, i, int(R[i])) for i in range(2)])).cuda()
    old = torch.from_numpy(np.concatenate([inputs.old_logp_noise(cfg, i, int(R[i])) for i in range(2)]) - 8.0).cuda()
    rewards = np.array([0.0, 1.0], dtype=np.float32)
    g = Guarded()
    dl = g.alloc("dlogits", (T, V), torch.bfloat16)
    lp = g.alloc("logp", (T,), torch.float32)
    cl = g.alloc("clipped", (T,), torch.uint8)
    loss = g.alloc("loss", (1,), torch.float32, zero=True)
    ws = g.alloc("loss workspace", (L.ls_grpo_workspace_bytes(T, V),), torch.uint8)
    L.ls_grpo_token_loss(lg, y, old, R, rewards, cfg.eps, 0, 2, loss, dlogits=dl, logp_out=lp, clipped_out=cl,
                         workspace=ws)
    L.ls_grpo_token_loss(lg, y, old, R, rewards, cfg.eps, 0, 2, loss, logp_out=lp, clipped_out=cl, workspace=ws,
                         scoring_only=True)
    dl2 = g.alloc("dlogits (no-workspace entry point)", (T, V), torch.bfloat16)
    L.ls_grpo_token_loss_noalloc(lg, y, old, R, rewards, cfg.eps, 0, 2, loss, dl2, logp_out=lp, clipped_out=cl)
    g.check()
    assert torch.equal(dl, dl2)


def test_lmhead_guard_bands():
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    cfg = inputs.replace(inputs.CONFIGS["tiny"], V=1000, seed=43)
    R = np.array([300, 31], dtype=np.int32)
    T, d = int(R.sum()), 40
    H = dev_bf16(np.concatenate([inputs.hidden(cfg, i, 0, int(R[i]), d) for i in range(2)]))
    W = dev_bf16(inputs.projection(cfg, d))
    y = torch.from_numpy(np.concatenate([inputs.targets(cfg, i, int(R[i])) for i in range(2)])).cuda()
    old = torch.full((T,), -7.0, dtype=torch.float32, device="cuda")
    rewards = np.array([1.0, 0.0], dtype=np.float32)
    g = Guarded()
    dH = g.alloc("dH", (T, d), torch.bfloat16)
    dW = g.alloc("dW", (cfg.V, d), torch.float32, zero=True)
    lp = g.alloc("logp", (T,), torch.float32)
    cl = g.alloc("clipped", (T,), torch.uint8)
    loss = g.alloc("loss", (1,), torch.float32, zero=True)
    ws = g.alloc("LM-head workspace", (L.ls_grpo_lmhead_workspace_bytes(T, cfg.V, d),), torch.uint8)
    L.ls_grpo_lmhead_loss(H, W, y, old, R, rewards, cfg.eps, 0, 2, loss, dW_accum=dW, dH=dH, logp_out=lp,
                          clipped_out=cl, workspace=ws)
    L.ls_grpo_lmhead_loss(H, W, y, old, R, rewards, cfg.eps, 0, 2, loss, logp_out=lp, clipped_out=cl,
                          workspace=ws, scoring_only=True)
    g.check()
    assert bool(torch.isfinite(dW).all()) and bool(torch.isfinite(dH.float()).all())


def _replay(cfg, R, rewards, first, last, dkp, dvp, loss):
    """Responses first .. last-1 of the group: forward, loss share, backward into the accumulators."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    cu = inputs.cu_seqlens(R)
    kp, vp = dev_bf16(inputs.prompt_k(cfg)), dev_bf16(inputs.prompt_v(cfg))
    for i in range(first, last):
        r0, r1 = int(cu[i]), int(cu[i + 1])
        r = r1 - r0
        q, ks = dev_bf16(inputs.suffix_q(cfg, r0, r1)), dev_bf16(inputs.suffix_k(cfg, r0, r1))
        vs, do = dev_bf16(inputs.suffix_v(cfg, r0, r1)), dev_bf16(inputs.suffix_do(cfg, r0, r1))
        lg = dev_bf16(inputs.logits(cfg, i, 0, r))
        y = torch.from_numpy(inputs.targets(cfg, i, r)).cuda()
        old = torch.from_numpy(inputs.old_logp_noise(cfg, i, r) - 8.0).cuda()
        lo = torch.empty(r, cfg.Hq, cfg.Dv, dtype=torch.bfloat16, device="cuda")
        o, lse = L.ls_replay_attn_fwd(q, ks, vs, kp, vp, [0, r], cfg.scale, o_lo=lo)
        L.ls_grpo_token_loss(lg, y, old, R, rewards, cfg.eps, i, 1, loss)
        L.ls_replay_attn_bwd(q, ks, vs, kp, vp, [0, r], o, lse, do, dkp, dvp, cfg.scale, o_lo=lo)
    torch.cuda.synchronize()


@pytest.mark.parametrize("D", [64, 128])
def test_checkpoint_resume_bitwise(D):
    import torch
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=8, Hkv=2, Dqk=D, Dv=D, P=3000, seed=44)
    R = np.array([64, 100, 77, 128], dtype=np.int32)
    rewards = inputs.rewards(inputs.replace(cfg, G=4))
    rewards[0] = 1.0 - rewards[1]

    def fresh():
        return (torch.zeros(cfg.P, cfg.Hkv, D, dtype=torch.float32, device="cuda"),
                torch.zeros(cfg.P, cfg.Hkv, D, dtype=torch.float32, device="cuda"),
                torch.zeros(1, dtype=torch.float32, device="cuda"))

    dkp, dvp, loss = fresh()
    _replay(cfg, R, rewards, 0, 4, dkp, dvp, loss)
    ref = [t.cpu().numpy() for t in (dkp, dvp, loss)]
    del dkp, dvp, loss

    dkp, dvp, loss = fresh()
    _replay(cfg, R, rewards, 0, 2, dkp, dvp, loss)
    saved = [t.cpu().numpy().copy() for t in (dkp, dvp, loss)]      # checkpoint at the response boundary
    del dkp, dvp, loss
    torch.cuda.empty_cache()
    dkp, dvp, loss = (torch.from_numpy(a).cuda() for a in saved)     # resume
    _replay(cfg, R, rewards, 2, 4, dkp, dvp, loss)
    got = [t.cpu().numpy() for t in (dkp, dvp, loss)]
    for name, a, b in zip(("dKp", "dVp", "loss"), got, ref):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name} differs after resume"
    assert np.any(ref[0] != 0) and ref[2][0] != 0
