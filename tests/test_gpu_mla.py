"""GPU parity of replay attention on latent-KV heads (Dqk 576, Dv 512, one kv head, V = the leading
512 dims of every K row) against the fp64 oracle (LongStraw study notes §2-1 step 4, §3-2 (2)/(4);
the latent-KV pages of the GLM run: the §3-1 overview table and §3-2 (1), (5)). Sizes span several query and key tiles with ragged tails."""
import numpy as np
import pytest

from prefix_shared_branch_amd import inputs
from tests.helpers import check_bf16_out, host_f64
from tests.test_gpu_attn import Case

pytestmark = pytest.mark.gpu

MLA = inputs.CONFIGS["mla"]


def _fwd_check(case, o, lse, ref):
    check_bf16_out(host_f64(o), ref["O"], "O")
    d = np.max(np.abs(host_f64(lse) - ref["LSE"]))
    assert d <= 1e-4, d


@pytest.mark.parametrize("P,lengths,seed", [(3000 + 17, [37, 130], 51), (0, [1, 70], 52), (64, [9], 53)])
def test_mla_forward(P, lengths, seed):
    case = Case(inputs.replace(MLA, P=P, seed=seed), lengths)
    o, lse = case.fwd()
    case.torch.cuda.synchronize()
    h = case.h
    from oracle import attn
    O, LSE = attn.replay_attn_fwd(h["Kp"], h["Vp"], h["Q"], h["Ks"], h["Vs"], case.cu, case.cfg.scale)
    _fwd_check(case, o, lse, dict(O=O, LSE=LSE))


def test_mla_forward_split_merge():
    """A long prompt and one short response: many prompt splits, merged by log-sum-exp."""
    from prefix_shared_branch_amd import lsreplay as L
    case = Case(inputs.replace(MLA, P=60000 + 5, seed=54), [20])
    desc = L.make_desc(case.q, case.kp, case.vp, case.ks, case.vs, case.cfg.scale)
    assert L.ls_replay_attn_workspace_bytes(desc, case.cu, 0) > 0
    o, lse = case.fwd()
    case.torch.cuda.synchronize()
    h = case.h
    from oracle import attn
    O, LSE = attn.replay_attn_fwd(h["Kp"], h["Vp"], h["Q"], h["Ks"], h["Vs"], case.cu, case.cfg.scale)
    _fwd_check(case, o, lse, dict(O=O, LSE=LSE))


def test_mla_unaliased_v_is_rejected():
    """The latent-KV kernels read V from the K rows: a separate V buffer is refused, not misread."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    case = Case(inputs.replace(MLA, P=100, seed=55), [5])
    vs = torch.empty(case.ks.shape[0], 1, 576, dtype=torch.bfloat16, device="cuda")[:, :, :512]
    vs.copy_(case.vs)
    with pytest.raises(L.LsError) as e:
        L.ls_replay_attn_fwd(case.q, case.ks, vs, case.kp, case.vp, case.cu, case.cfg.scale)
    assert e.value.code == L.LS_ERR_UNSUPPORTED


@pytest.mark.parametrize("P,lengths,seed", [(3000 + 17, [37, 130], 56), (64, [9, 2], 57), (500, [5, 0, 20], 61)])
def test_mla_backward_exact(P, lengths, seed):
    """One call over several responses: dQ, response-key dK/dV, and the prompt accumulators."""
    from tests.test_gpu_attn import _check_all
    case = Case(inputs.replace(MLA, P=P, seed=seed), lengths)
    t = case.torch
    dkp, dvp = case.accums()
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
    t.cuda.synchronize()
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp), case.oracle())


def test_mla_backward_no_prompt():
    from tests.test_gpu_attn import _check_all
    case = Case(inputs.replace(MLA, P=0, seed=58), [1, 70])
    o, lse = case.fwd()
    dq, dks, dvs = case.bwd(o, lse)
    case.torch.cuda.synchronize()
    _check_all(dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs), case.oracle(accumulate=False), literal_abs=False)


def test_mla_serial_replay_and_split_dq():
    """Serial replay (prompt gradients accumulated over calls) over a prompt long enough for split-K
    in the forward and dQ kernels."""
    from tests.test_gpu_attn import _check_all, _serial
    case = Case(inputs.replace(MLA, P=30000 + 3, seed=59), [20, 45])
    _check_all(_serial(case), case.oracle())


def test_mla_blockwise_replay():
    from tests.test_gpu_block import _blockwise, _check
    case = Case(inputs.replace(MLA, P=2000, seed=60), [150])
    _check(_blockwise(case, [0, 1, 70, 150]), case.oracle())


def test_mla_full_prompt_sampled_rows_and_column_sums():
    """P = 2,097,152 latent rows and the first response at its full length, in the launch
    configuration the benchmark times (one call per response, exact prompt gradients). O, LSE and
    dQ on sampled rows and heads (each row and head depends on that row and head alone); the
    value-gradient column sums sum_j dV_P[j] + sum_s dVs[s] = sum_t sum_h dO[t, h] (softmax weights
    sum to one) over all heads."""
    import torch
    from oracle import attn
    from prefix_shared_branch_amd import lsreplay as L
    from tests.helpers import dev_bf16
    cfg = MLA
    f64 = inputs.bf16_bits_to_f64
    r = int(inputs.response_lengths(cfg)[0])
    kp_bits = inputs.prompt_k(cfg)
    kp = dev_bf16(kp_bits)
    q_b, ks_b, do_b = inputs.suffix_q(cfg, 0, r), inputs.suffix_k(cfg, 0, r), inputs.suffix_do(cfg, 0, r)
    q, ks, do = dev_bf16(q_b), dev_bf16(ks_b), dev_bf16(do_b)
    vp, vs = kp[:, :, :cfg.Dv], ks[:, :, :cfg.Dv]
    dkp = torch.zeros(cfg.P, 1, cfg.Dqk, dtype=torch.float32, device="cuda")
    dvp = torch.zeros(cfg.P, 1, cfg.Dv, dtype=torch.float32, device="cuda")
    lo = torch.empty(r, cfg.Hq, cfg.Dv, dtype=torch.bfloat16, device="cuda")
    o, lse = L.ls_replay_attn_fwd(q, ks, vs, kp, vp, [0, r], cfg.scale, o_lo=lo)
    dq, dks, dvs = L.ls_replay_attn_bwd(q, ks, vs, kp, vp, [0, r], o, lse, do, dkp, dvp, cfg.scale, o_lo=lo)
    torch.cuda.synchronize()
    # the oracle at full P for two of the 16 query heads (heads share the one latent kv head)
    hs = [0, cfg.Hq - 1]
    Kp = f64(kp_bits)
    del kp_bits
    Ks, Q, dO = f64(ks_b), f64(q_b)[:, hs, :], f64(do_b)
    rows = np.array([0, r - 1])
    O, LSE = attn.replay_attn_fwd(Kp, Kp[:, :, :cfg.Dv], Q, Ks, Ks[:, :, :cfg.Dv], [0, r], cfg.scale, rows=rows)
    check_bf16_out(host_f64(o[rows][:, hs]), O[rows], "O rows")
    d = host_f64(lse)[hs][:, rows] - LSE[:, rows]
    assert np.max(np.abs(d)) <= 1e-4, d
    dQ = attn.replay_attn_bwd_rows(Kp, Kp[:, :, :cfg.Dv], Q, Ks, Ks[:, :, :cfg.Dv], dO[:, hs, :], [0, r], cfg.scale,
                                   rows)
    check_bf16_out(host_f64(dq[rows][:, hs]), dQ, "dQ rows")
    # every head: value-gradient column sums
    want = dO.sum(axis=(0, 1))
    have = (dvp.double().sum(dim=(0, 1)) + dvs.double().sum(dim=(0, 1))).cpu().numpy()
    rel = np.linalg.norm(have - want) / np.linalg.norm(want)
    assert rel <= 1e-3, rel
