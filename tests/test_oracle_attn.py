"""Pins of the replay-attention oracle against things other than itself (CPU only).

Sources of truth: textbook causal attention on the concatenated [prompt; response]
sequence (a separate numpy routine), torch float64 SDPA + autograd, central finite
differences, closed forms (zero keys, constant values, hand-worked example), and the
serial-replay invariant of the LongStraw study notes (§2-1 step 4: the prompt-side
gradient summed over serially replayed responses equals the whole-group backward).
"""
import json
import os

import numpy as np
import pytest

from oracle import attn, brute, fd
from prefix_shared_branch_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make_case(seed, P, lengths, Hq, Hkv, D, Dv=None):
    Dv = D if Dv is None else Dv
    g = np.random.default_rng(seed)
    T = int(np.sum(lengths))
    return dict(Kp=g.standard_normal((P, Hkv, D)), Vp=g.standard_normal((P, Hkv, Dv)),
                Q=g.standard_normal((T, Hq, D)), Ks=g.standard_normal((T, Hkv, D)),
                Vs=g.standard_normal((T, Hkv, Dv)), dO=g.standard_normal((T, Hq, Dv)),
                cu=inputs.cu_seqlens(lengths))


@pytest.mark.parametrize("P,lengths,Hq,Hkv,D", [(7, [5, 3], 4, 2, 8), (0, [6], 2, 1, 4), (16, [1, 9, 4], 6, 3, 5)])
def test_fwd_matches_causal_concat(P, lengths, Hq, Hkv, D):
    c = make_case(3, P, lengths, Hq, Hkv, D)
    scale = 0.37
    O, LSE = attn.replay_attn_fwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["cu"], scale)
    for i in range(len(lengths)):
        r0, r1 = c["cu"][i], c["cu"][i + 1]
        Ob, Lb = brute.causal_concat_fwd(c["Kp"], c["Vp"], c["Q"][r0:r1], c["Ks"][r0:r1], c["Vs"][r0:r1], scale)
        np.testing.assert_allclose(O[r0:r1], Ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(LSE[:, r0:r1], Lb, rtol=1e-12, atol=1e-12)


def test_fwd_bwd_match_torch_sdpa():
    P, lengths, Hq, Hkv, D = 11, [7, 4], 6, 2, 8
    c = make_case(5, P, lengths, Hq, Hkv, D)
    scale = 1 / np.sqrt(D)
    O, _ = attn.replay_attn_fwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["cu"], scale)
    dKp = np.zeros_like(c["Kp"])
    dVp = np.zeros_like(c["Vp"])
    dQ, dKs, dVs = attn.replay_attn_bwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], c["cu"], scale, dKp, dVp)
    sum_dKp = np.zeros_like(dKp)
    sum_dVp = np.zeros_like(dVp)
    for i in range(len(lengths)):
        r0, r1 = c["cu"][i], c["cu"][i + 1]
        Ot, dQt, dKpt, dVpt, dKst, dVst = brute.torch_concat_fwd_bwd(
            c["Kp"], c["Vp"], c["Q"][r0:r1], c["Ks"][r0:r1], c["Vs"][r0:r1], c["dO"][r0:r1], scale)
        np.testing.assert_allclose(O[r0:r1], Ot, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dQ[r0:r1], dQt, rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dKs[r0:r1], dKst, rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dVs[r0:r1], dVst, rtol=1e-10, atol=1e-11)
        sum_dKp += dKpt
        sum_dVp += dVpt
    np.testing.assert_allclose(dKp, sum_dKp, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dVp, sum_dVp, rtol=1e-10, atol=1e-11)


def test_serial_replay_equals_tree_batched_backward():
    """Sum over serially replayed responses of the prompt-side gradient == whole-group batched backward."""
    P, lengths, Hq, Hkv, D = 9, [4, 6, 3, 5], 4, 2, 6
    c = make_case(7, P, lengths, Hq, Hkv, D)
    scale = 0.41
    dKp = np.zeros_like(c["Kp"])
    dVp = np.zeros_like(c["Vp"])
    dQ = np.zeros_like(c["Q"])
    dKs = np.zeros_like(c["Ks"])
    dVs = np.zeros_like(c["Vs"])
    for i in range(len(lengths)):          # one response per call, accumulating in place
        r0, r1 = c["cu"][i], c["cu"][i + 1]
        cu1 = np.array([0, r1 - r0])
        q, ks, vs, do = (c[n][r0:r1] for n in ("Q", "Ks", "Vs", "dO"))
        dq, dks, dvs = attn.replay_attn_bwd(c["Kp"], c["Vp"], q, ks, vs, do, cu1, scale, dKp, dVp)
        dQ[r0:r1], dKs[r0:r1], dVs[r0:r1] = dq, dks, dvs
    Ob, dQb, dKpb, dVpb, dKsb, dVsb = brute.torch_tree_batch_grads(
        c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], c["cu"], scale)
    np.testing.assert_allclose(dKp, dKpb, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dVp, dVpb, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dQ, dQb, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dKs, dKsb, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dVs, dVsb, rtol=1e-10, atol=1e-12)
    O, _ = attn.replay_attn_fwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["cu"], scale)
    np.testing.assert_allclose(O, Ob, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("R", [3, 5])
def test_bwd_finite_differences(R):
    """Micro shape: Hq 2, Hkv 1, D 4, P 6; every gradient vs central differences of sum(O * dO)."""
    P, Hq, Hkv, D = 6, 2, 1, 4
    c = make_case(21 + R, P, [R], Hq, Hkv, D)
    scale = 0.5
    cu = c["cu"]

    def f_of(name):
        def f(x):
            args = {k: c[k] for k in ("Kp", "Vp", "Q", "Ks", "Vs")}
            args[name] = x
            O, _ = attn.replay_attn_fwd(args["Kp"], args["Vp"], args["Q"], args["Ks"], args["Vs"], cu, scale)
            return float(np.sum(O * c["dO"]))
        return f

    dKp = np.zeros_like(c["Kp"])
    dVp = np.zeros_like(c["Vp"])
    dQ, dKs, dVs = attn.replay_attn_bwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], cu, scale, dKp, dVp)
    for name, got in (("Q", dQ), ("Ks", dKs), ("Vs", dVs), ("Kp", dKp), ("Vp", dVp)):
        num = fd.grad(f_of(name), c[name])
        err = np.max(np.abs(num - got)) / max(1e-30, np.max(np.abs(num)))
        assert err < 1e-7, (name, err)


def test_zero_keys_closed_form():
    """K == 0: every visible key gets weight 1/(P+t+1); LSE = log(P+t+1); dV_P[j] = sum_h sum_t dO/(P+t+1)."""
    P, lengths, Hq, Hkv, D = 10, [6, 4], 4, 2, 5
    c = make_case(9, P, lengths, Hq, Hkv, D)
    Kp0, Ks0 = np.zeros_like(c["Kp"]), np.zeros_like(c["Ks"])
    O, LSE = attn.replay_attn_fwd(Kp0, c["Vp"], c["Q"], Ks0, c["Vs"], c["cu"], 0.3)
    dKp = np.zeros_like(c["Kp"])
    dVp = np.zeros_like(c["Vp"])
    attn.replay_attn_bwd(Kp0, c["Vp"], c["Q"], Ks0, c["Vs"], c["dO"], c["cu"], 0.3, dKp, dVp)
    g = Hq // Hkv
    exp_dVp = np.zeros_like(dVp)
    for i in range(len(lengths)):
        r0, r1 = c["cu"][i], c["cu"][i + 1]
        for t in range(r1 - r0):
            n = P + t + 1
            for h in range(Hq):
                k = h // g
                want = (c["Vp"][:, k].sum(0) + c["Vs"][r0:r0 + t + 1, k].sum(0)) / n
                np.testing.assert_allclose(O[r0 + t, h], want, rtol=1e-12, atol=1e-13)
                assert abs(LSE[h, r0 + t] - np.log(n)) < 1e-12
                exp_dVp[:, k] += c["dO"][r0 + t, h] / n
    np.testing.assert_allclose(dVp, exp_dVp, rtol=1e-12, atol=1e-13)


def test_constant_values():
    """All value rows equal to c => O == c exactly for any scores; zero-mean dO then gives dQ = dK = 0."""
    P, lengths, Hq, Hkv, D = 12, [5], 2, 1, 4
    c = make_case(11, P, lengths, Hq, Hkv, D)
    cv = np.array([0.5, -1.25, 2.0, 3.0])
    Vp = np.broadcast_to(cv, c["Vp"].shape).copy()
    Vs = np.broadcast_to(cv, c["Vs"].shape).copy()
    O, _ = attn.replay_attn_fwd(c["Kp"], Vp, c["Q"], c["Ks"], Vs, c["cu"], 0.7)
    np.testing.assert_allclose(O, np.broadcast_to(cv, O.shape), rtol=1e-13, atol=1e-13)
    dQ, dKs, _ = attn.replay_attn_bwd(c["Kp"], Vp, c["Q"], c["Ks"], Vs, c["dO"], c["cu"], 0.7)
    assert np.max(np.abs(dQ)) < 1e-12 and np.max(np.abs(dKs)) < 1e-12


def test_hand_worked_example():
    """P=1, R=2, one head, D=1, scale 1 (derivation in tests/golden/hand_attn.json)."""
    with open(os.path.join(GOLDEN, "hand_attn.json")) as f:
        gd = json.load(f)
    a = {k: np.array(v, dtype=np.float64) for k, v in gd["inputs"].items()}
    O, LSE = attn.replay_attn_fwd(a["Kp"], a["Vp"], a["Q"], a["Ks"], a["Vs"], [0, 2], 1.0)
    e = np.e
    want_O = [2 * e / (e + 1), 2.0]          # row 0 sees (Kp, Ks0); row 1 sees all three with equal scores
    want_L = [np.log(e + 1), np.log(3.0)]
    np.testing.assert_allclose(O[:, 0, 0], want_O, rtol=1e-14)
    np.testing.assert_allclose(LSE[0], want_L, rtol=1e-14)
    np.testing.assert_allclose(O[:, 0, 0], gd["O"], rtol=1e-12)
    np.testing.assert_allclose(LSE[0], gd["LSE"], rtol=1e-12)


def test_response_only_mode_leaves_prompt_side_alone():
    P, lengths, Hq, Hkv, D = 8, [5], 4, 2, 4
    c = make_case(13, P, lengths, Hq, Hkv, D)
    dKp = np.zeros_like(c["Kp"])
    dVp = np.zeros_like(c["Vp"])
    a = attn.replay_attn_bwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], c["cu"], 0.5, dKp, dVp)
    b = attn.replay_attn_bwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], c["cu"], 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert np.any(dKp != 0)
    with pytest.raises(ValueError):
        attn.replay_attn_bwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], c["cu"], 0.5, dKp, None)


def test_selected_rows_match_full():
    P, lengths, Hq, Hkv, D = 20, [7, 9], 4, 1, 6
    c = make_case(17, P, lengths, Hq, Hkv, D)
    O, LSE = attn.replay_attn_fwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["cu"], 0.4)
    rows = [0, 3, 8, 15]
    Or, Lr = attn.replay_attn_fwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["cu"], 0.4, rows=rows)
    np.testing.assert_array_equal(Or[rows], O[rows])
    np.testing.assert_array_equal(Lr[:, rows], LSE[:, rows])
    dQ, _, _ = attn.replay_attn_bwd(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], c["cu"], 0.4)
    dQr = attn.replay_attn_bwd_rows(c["Kp"], c["Vp"], c["Q"], c["Ks"], c["Vs"], c["dO"], c["cu"], 0.4, rows)
    np.testing.assert_allclose(dQr, dQ[rows], rtol=1e-12, atol=1e-13)


def test_latent_kv_aliasing():
    """Latent KV: V is a strided view of the first Dv dims of K; same result as an explicit copy."""
    P, lengths, Hq, D, Dv = 10, [6], 4, 12, 8
    c = make_case(19, P, lengths, Hq, 1, D, Dv)
    Vp_view, Vs_view = c["Kp"][:, :, :Dv], c["Ks"][:, :, :Dv]
    O1, L1 = attn.replay_attn_fwd(c["Kp"], Vp_view, c["Q"], c["Ks"], Vs_view, c["cu"], 0.3)
    O2, L2 = attn.replay_attn_fwd(c["Kp"], Vp_view.copy(), c["Q"], c["Ks"], Vs_view.copy(), c["cu"], 0.3)
    np.testing.assert_array_equal(O1, O2)
    Ob, Lb = brute.causal_concat_fwd(c["Kp"], Vp_view, c["Q"], c["Ks"], Vs_view, 0.3)
    np.testing.assert_allclose(O1, Ob, rtol=1e-12, atol=1e-13)
