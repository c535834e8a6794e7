"""GPU parity of blockwise suffix replay (ls_replay_attn_fwd_block / ls_replay_attn_bwd_block)
against the fp64 oracle of the whole response.

One response is replayed in blocks of query rows (LongStraw study notes §3-2, blockwise suffix
replay): block rows q0 .. q1-1 attend to the prompt and causally to the response's keys 0 .. q1-1.
Attention rows are independent and gradients are sums over rows, so the blocks together must give
the full response's O, LSE and dQ row by row, and its key gradients once every block's share is
added. The oracle is the unblocked whole-response replay."""
import numpy as np
import pytest

from prefix_shared_branch_amd import inputs
from tests.helpers import check_bf16_out, check_fp32_accum, host_f64
from tests.test_gpu_attn import Case

pytestmark = pytest.mark.gpu


def _blockwise(case, bounds, exact=True):
    from prefix_shared_branch_amd import lsreplay as L
    t = case.torch
    cfg = case.cfg
    R = int(case.lengths[0])
    dks = t.zeros(R, cfg.Hkv, cfg.Dqk, dtype=t.float32, device="cuda")
    dvs = t.zeros(R, cfg.Hkv, cfg.Dv, dtype=t.float32, device="cuda")
    dkp, dvp = case.accums() if exact else (None, None)
    outs = {"O": [], "LSE": [], "dQ": []}
    for q0, q1 in zip(bounds[:-1], bounds[1:]):
        q, ks, vs, do = case.q[q0:q1], case.ks[:q1], case.vs[:q1], case.do[q0:q1]
        lo = t.empty(q1 - q0, cfg.Hq, cfg.Dv, dtype=t.bfloat16, device="cuda")
        o, lse = L.ls_replay_attn_fwd_block(q, ks, vs, case.kp, case.vp, q0, cfg.scale, o_lo=lo)
        dq = L.ls_replay_attn_bwd_block(q, ks, vs, case.kp, case.vp, q0, o, lse, do, dks[:q1], dvs[:q1], dkp, dvp,
                                        cfg.scale, o_lo=lo)
        outs["O"].append(o)
        outs["LSE"].append(lse)
        outs["dQ"].append(dq)
    t.cuda.synchronize()
    got = {k: t.cat(v, dim=1 if k == "LSE" else 0) for k, v in outs.items()}
    got.update(dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp)
    return got


def _check(got, ref, exact=True, literal_abs=True):
    check_bf16_out(host_f64(got["O"]), ref["O"], "O", literal_abs=literal_abs)
    lse = host_f64(got["LSE"])
    assert np.max(np.abs(lse - ref["LSE"])) <= 1e-4, np.max(np.abs(lse - ref["LSE"]))
    check_bf16_out(host_f64(got["dQ"]), ref["dQ"], "dQ", literal_abs=literal_abs)
    # Response-key gradients: the unblocked call returns these in bf16 and they are checked at the
    # bf16-output bar there; the block call keeps them in fp32 only so that blocks add without a
    # bf16 rounding per block. Each key sums over few rows (causal), so the fp16 operand rounding of
    # the dK/dV products does not average down as it does for the prompt accumulators.
    check_bf16_out(host_f64(got["dKs"]), ref["dKs"], "dKs", literal_abs=literal_abs)
    check_bf16_out(host_f64(got["dVs"]), ref["dVs"], "dVs", literal_abs=literal_abs)
    if exact:
        check_fp32_accum(host_f64(got["dKp"]), ref["dKp"], "dKp")
        check_fp32_accum(host_f64(got["dVp"]), ref["dVp"], "dVp")


@pytest.mark.parametrize("D,P,R,bounds", [
    (64, 1000, 300, [0, 1, 130, 300]),          # a one-row block, then ragged blocks
    (128, 5000, 700, [0, 256, 257, 500, 700]),  # tile-aligned and off-by-one boundaries
    (128, 0, 200, [0, 64, 200]),                # no prompt: plain causal attention in blocks
])
def test_blocks_match_whole_response(D, P, R, bounds):
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=8, Hkv=2, Dqk=D, Dv=D, P=P, seed=41)
    case = Case(cfg, [R])
    exact = P > 0
    _check(_blockwise(case, bounds, exact), case.oracle(accumulate=exact), exact)


def test_single_block_equals_unblocked_call():
    """One block covering the whole response is the ordinary call, bit for bit in O, LSE and dQ."""
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=8, Hkv=2, Dqk=128, Dv=128, P=3000, seed=42)
    case = Case(cfg, [333])
    t = case.torch
    got = _blockwise(case, [0, 333])
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    assert t.equal(got["O"], o) and t.equal(got["LSE"], lse) and t.equal(got["dQ"], dq)
    assert t.equal(got["dKp"], dkp) and t.equal(got["dVp"], dvp)
