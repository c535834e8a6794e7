"""GPU parity of ls_replay_attn_fwd / ls_replay_attn_bwd against the fp64 oracle.

Replay semantics (LongStraw study notes §2-1 step 4, §3-2 (2)/(4)): response queries attend to
the resident prompt K/V and, causally, to their own K/V; serial replay adds each response's
prompt-side gradient into fp32 accumulators owned by the prompt pages. Every case runs the
kernels through the C ABI on seeded bf16 inputs and compares with the oracle element by element.
"""
import numpy as np
import pytest

from oracle import attn
from prefix_shared_branch_amd import inputs
from tests.helpers import check_bf16_out, check_fp32_accum, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


class Case:
    """Seeded inputs of one config with explicit response lengths (packed)."""

    def __init__(self, cfg, lengths, residual=True):
        import torch
        self.cfg = cfg
        self.residual = residual  # pass the forward's rounding residual of O to the backward
        self.lengths = np.asarray(lengths, dtype=np.int32)
        self.cu = inputs.cu_seqlens(self.lengths)
        T = int(self.cu[-1])
        kp = inputs.prompt_k(cfg)
        vp = inputs.prompt_v(cfg) if not cfg.mla else None
        q, ks, do = inputs.suffix_q(cfg, 0, T), inputs.suffix_k(cfg, 0, T), inputs.suffix_do(cfg, 0, T)
        vs = inputs.suffix_v(cfg, 0, T) if not cfg.mla else None
        self.h = dict(Kp=inputs.bf16_bits_to_f64(kp), Q=inputs.bf16_bits_to_f64(q), Ks=inputs.bf16_bits_to_f64(ks),
                      dO=inputs.bf16_bits_to_f64(do))
        self.kp, self.q, self.ks, self.do = dev_bf16(kp), dev_bf16(q), dev_bf16(ks), dev_bf16(do)
        if cfg.mla:
            self.vp, self.vs = self.kp[:, :, :cfg.Dv], self.ks[:, :, :cfg.Dv]
            self.h["Vp"], self.h["Vs"] = self.h["Kp"][:, :, :cfg.Dv], self.h["Ks"][:, :, :cfg.Dv]
        else:
            self.vp, self.vs = dev_bf16(vp), dev_bf16(vs)
            self.h["Vp"], self.h["Vs"] = inputs.bf16_bits_to_f64(vp), inputs.bf16_bits_to_f64(vs)
        self.torch = torch

    def fwd(self, cu=None, sl=slice(None)):
        """Forward; with residual, O carries its rounding residual as the attribute o_lo."""
        from prefix_shared_branch_amd import lsreplay as L
        cu = self.cu if cu is None else cu
        q = self.q[sl]
        lo = self.torch.empty(q.shape[0], self.cfg.Hq, self.cfg.Dv, dtype=self.torch.bfloat16,
                              device="cuda") if self.residual else None
        o, lse = L.ls_replay_attn_fwd(q, self.ks[sl], self.vs[sl], self.kp, self.vp, cu, self.cfg.scale, o_lo=lo)
        o.o_lo = lo
        return o, lse

    def bwd(self, o, lse, dkp=None, dvp=None, cu=None, sl=slice(None)):
        from prefix_shared_branch_amd import lsreplay as L
        cu = self.cu if cu is None else cu
        return L.ls_replay_attn_bwd(self.q[sl], self.ks[sl], self.vs[sl], self.kp, self.vp, cu, o, lse, self.do[sl],
                                    dkp, dvp, self.cfg.scale, o_lo=getattr(o, "o_lo", None))

    def accums(self):
        t = self.torch
        P, Hkv = self.cfg.P, self.cfg.Hkv
        return (t.zeros(P, Hkv, self.cfg.Dqk, dtype=t.float32, device="cuda"),
                t.zeros(P, Hkv, self.cfg.Dv, dtype=t.float32, device="cuda"))

    def oracle(self, accumulate=True):
        h = self.h
        O, LSE = attn.replay_attn_fwd(h["Kp"], h["Vp"], h["Q"], h["Ks"], h["Vs"], self.cu, self.cfg.scale)
        dKp = np.zeros_like(h["Kp"]) if accumulate else None
        dVp = np.zeros(h["Vp"].shape) if accumulate else None
        dQ, dKs, dVs = attn.replay_attn_bwd(h["Kp"], h["Vp"], h["Q"], h["Ks"], h["Vs"], h["dO"], self.cu,
                                            self.cfg.scale, dKp, dVp)
        return dict(O=O, LSE=LSE, dQ=dQ, dKs=dKs, dVs=dVs, dKp=dKp, dVp=dVp)


def _check_all(got, ref, literal_abs=True):
    check_bf16_out(host_f64(got["O"]), ref["O"], "O", literal_abs=literal_abs)
    lse = host_f64(got["LSE"])
    assert np.max(np.abs(lse - ref["LSE"])) <= 1e-4, np.max(np.abs(lse - ref["LSE"]))
    check_bf16_out(host_f64(got["dQ"]), ref["dQ"], "dQ", literal_abs=literal_abs)
    check_bf16_out(host_f64(got["dKs"]), ref["dKs"], "dKs", literal_abs=literal_abs)
    check_bf16_out(host_f64(got["dVs"]), ref["dVs"], "dVs", literal_abs=literal_abs)
    if ref.get("dKp") is not None and ref["dKp"].size:
        check_fp32_accum(host_f64(got["dKp"]), ref["dKp"], "dKp")
        check_fp32_accum(host_f64(got["dVp"]), ref["dVp"], "dVp")


def _serial(case):
    """Serial replay: one call per response, prompt gradients accumulated in place."""
    t = case.torch
    dkp, dvp = case.accums()
    outs = {k: [] for k in ("O", "LSE", "dQ", "dKs", "dVs")}
    for i in range(len(case.lengths)):
        r0, r1 = int(case.cu[i]), int(case.cu[i + 1])
        cu1 = [0, r1 - r0]
        o, lse = case.fwd(cu1, slice(r0, r1))
        dq, dks, dvs = case.bwd(o, lse, dkp, dvp, cu1, slice(r0, r1))
        for k, v in zip(("O", "LSE", "dQ", "dKs", "dVs"), (o, lse, dq, dks, dvs)):
            outs[k].append(v)
    t.cuda.synchronize()
    got = {k: t.cat(v, dim=1 if k == "LSE" else 0) for k, v in outs.items()}
    got["dKp"], got["dVp"] = dkp, dvp
    return got


def test_tiny_full_group_serial_replay():
    case = Case(inputs.CONFIGS["tiny"], inputs.response_lengths(inputs.CONFIGS["tiny"]))
    _check_all(_serial(case), case.oracle())


@pytest.mark.parametrize("D", [64, 128])
def test_ragged_multi_response_call(D):
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=6, Hkv=2, Dqk=D, Dv=D, P=1000, seed=31)
    case = Case(cfg, [1, 37, 130])
    t = case.torch
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp), case.oracle())


@pytest.mark.parametrize("P", [1, 255, 257, 511])
def test_prompt_dkdv_tile_edges(P):
    """Head dim 128, serial calls of 1, 8 and 9 tokens (4, 32 and 36 packed rows: one, one and two
    32-row steps, fewer than the load ring's depth) over prompts of 1, 255, 257 and 511 keys, whose
    last 256-key tile holds 1 or 255 keys: whole waves, and single 32-key blocks of a wave, without
    a valid key."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=8, Hkv=2, Dqk=128, Dv=128, P=P, seed=39)
    case = Case(cfg, [1, 8, 9])
    _check_all(_serial(case), case.oracle(), literal_abs=False)


@pytest.mark.parametrize("Hq,Hkv", [(16, 1), (16, 2)])
def test_wide_gqa_groups(Hq, Hkv):
    """Head dim 128 with 16 and 8 query heads per kv head: many packed rows per token, so a short
    response already spans several 32-row steps of the prompt dK/dV sweep and several dQ row tiles."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=Hq, Hkv=Hkv, Dqk=128, Dv=128, P=700, seed=40)
    case = Case(cfg, [3, 41])
    _check_all(_serial(case), case.oracle(), literal_abs=False)


def test_no_prompt_is_plain_causal():
    cfg = inputs.replace(inputs.CONFIGS["tiny"], P=0, seed=32)
    case = Case(cfg, [70, 5])
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse)
    case.torch.cuda.synchronize()
    # no prompt: gradients of order 1-4, so only the scale-aware bounds apply
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs), case.oracle(accumulate=False), literal_abs=False)


def test_split_k_merge_path():
    """Few query tiles and a long prompt: the planner picks many splits (LSE merge, dQ partial sums)."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=8, Hkv=2, Dqk=128, Dv=128, P=20000 + 37, seed=33)
    case = Case(cfg, [50])
    from prefix_shared_branch_amd import lsreplay as L
    desc = L.make_desc(case.q, case.kp, case.vp, case.ks, case.vs, cfg.scale)
    assert L.ls_replay_attn_workspace_bytes(desc, case.cu, 0) > 0      # split partials in use
    t = case.torch
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp), case.oracle())


def test_serial_equals_batched_call_and_modes():
    """One call over the whole group == G serial calls (accumulators to 1e-6 rel); response-only
    mode leaves accumulators untouched and gives bitwise the same dQ/dKs/dVs; K/V never written."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], seed=34)
    case = Case(cfg, [64, 100, 77, 128])
    t = case.torch
    kp0, vp0 = case.kp.clone(), case.vp.clone()
    ser = _serial(case)
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    snap_k, snap_v = dkp.clone(), dvp.clone()
    dq2, dks2, dvs2 = case.bwd(o, lse)                       # response-only closure
    t.cuda.synchronize()
    for a, b in ((dkp, ser["dKp"]), (dvp, ser["dVp"])):
        rel = (a - b).norm().item() / b.norm().item()
        assert rel <= 1e-6, rel
    assert t.equal(o, ser["O"]) and t.equal(lse, ser["LSE"])
    assert t.equal(dq, dq2) and t.equal(dks, dks2) and t.equal(dvs, dvs2)
    assert t.equal(dkp, snap_k) and t.equal(dvp, snap_v)
    assert t.equal(case.kp, kp0) and t.equal(case.vp, vp0)


def test_bitwise_determinism():
    cfg = inputs.replace(inputs.CONFIGS["tiny"], P=5000, seed=35)
    case = Case(cfg, [90, 33])
    t = case.torch
    res = []
    for _ in range(2):
        dkp, dvp = case.accums()
        o, lse = case.fwd()
        dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
        res.append((o, lse, dq, dks, dvs, dkp, dvp))
    t.cuda.synchronize()
    for a, b in zip(*res):
        assert t.equal(a, b)


def test_mid_shape_short_response():
    """Mid config (Hq 32 / Hkv 8, D 128, P 32768) with its first 256 response rows: an exact sub-problem."""
    case = Case(inputs.CONFIGS["mid"], [256])
    t = case.torch
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp), case.oracle())


def test_kernel_timer_counts_launches():
    """The instrumentation timer brackets each launch of the armed kernel and nothing else."""
    from prefix_shared_branch_amd import lsreplay as L
    case = Case(inputs.CONFIGS["tiny"], [70, 90])
    t = case.torch
    dkp, dvp = case.accums()
    L.ls_kernel_timer_start(L.LS_KERNEL_DKDV_PROMPT)
    o, lse = case.fwd()
    case.bwd(o, lse, dkp, dvp)      # exact mode: one prompt dK/dV launch
    case.bwd(o, lse)                # response-only: no prompt dK/dV launch
    case.bwd(o, lse, dkp, dvp)
    ms, n = L.ls_kernel_timer_stop()
    t.cuda.synchronize()
    assert n == 2 and ms > 0.0, (ms, n)
    L.ls_kernel_timer_start(L.LS_KERNEL_ATTN_FWD)
    case.fwd()
    ms, n = L.ls_kernel_timer_stop()
    assert n == 1 and ms > 0.0, (ms, n)


@pytest.mark.parametrize("do_scale,q_scale", [(3e-7, 1.0), (5e4, 1.0), (1.0, 0.05), (0.0, 1.0)])
def test_backward_operand_scaling(do_scale, q_scale):
    """The dK/dV products run in fp16 on operands scaled by per-call powers of two; gradients of
    realistic (tiny) or large magnitude, small queries and an all-zero dO must keep the accumulator
    bar. Scaled inputs are re-rounded to bf16 and the oracle sees those values."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], P=3000, seed=36)
    case = Case(cfg, [77, 120])

    def rescale(bits, f):
        return inputs.f32_to_bf16_bits((inputs.bf16_bits_to_f32(bits) * np.float32(f)).astype(np.float32))

    T = int(case.cu[-1])
    do_bits = rescale(inputs.suffix_do(cfg, 0, T), do_scale)
    q_bits = rescale(inputs.suffix_q(cfg, 0, T), q_scale)
    case.do, case.h["dO"] = dev_bf16(do_bits), inputs.bf16_bits_to_f64(do_bits)
    case.q, case.h["Q"] = dev_bf16(q_bits), inputs.bf16_bits_to_f64(q_bits)
    t = case.torch
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    ref = case.oracle()
    if do_scale == 0.0:
        for x in (dkp, dvp, dq, dks, dvs):
            assert not bool(x.any()), "a zero dO must give exactly zero gradients"
        return
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp), ref, literal_abs=False)


def test_output_rounding_residual():
    """O_lo holds the fp32 output's rounding residual: at most half a bf16 step of O, and O + O_lo
    is closer to the fp64 output than O alone (long prompt: the fp32 sum is far below a bf16 step)."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=8, Hkv=2, Dqk=128, Dv=128, P=5000, seed=37)
    case = Case(cfg, [70, 130])
    o, _ = case.fwd()
    case.torch.cuda.synchronize()
    hi, lo = host_f64(o), host_f64(o.o_lo)
    ref = case.oracle(accumulate=False)["O"]
    # one bf16 step at |O| in [2^e, 2^(e+1)) is 2^(e - 7)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(hi), 1e-30))) - 7)
    assert np.all(np.abs(lo) <= step / 2 * (1 + 2 ** -7))
    for h in range(cfg.Hq):
        e_hi = np.linalg.norm(hi[:, h] - ref[:, h])
        e_sum = np.linalg.norm(hi[:, h] + lo[:, h] - ref[:, h])
        assert e_sum <= 0.5 * e_hi, (h, e_sum, e_hi)


def test_backward_without_output_residual():
    """O_lo is optional: Delta from the bf16 O alone keeps the bars at a prompt of a thousand keys."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], P=1000, seed=38)
    case = Case(cfg, [40, 200], residual=False)
    t = case.torch
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    assert o.o_lo is None
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp), case.oracle())


@pytest.mark.parametrize("base,scale", [("tiny", 0.01), ("tiny", 1.0), ("mid", 0.01), ("mid", 1.0)])
def test_softmax_scale_extremes(base, scale):
    """A caller-chosen softmax scale far from 1/sqrt(D): nearly flat (0.01) and nearly one-hot (1.0)
    attention. The dK/dV kernel takes LSE and Delta as three-part bf16 row terms inside its MFMAs,
    with LSE divided by the scale, so both ends of the scale range check those terms."""
    import dataclasses
    import types
    cfg = inputs.replace(inputs.CONFIGS[base], P=2000, seed=41)
    case = Case(cfg, [70, 129])
    case.cfg = types.SimpleNamespace(**dataclasses.asdict(cfg), scale=scale)
    t = case.torch
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp), case.oracle(), literal_abs=False)
