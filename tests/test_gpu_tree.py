"""Replay over a two-level prefix tree with the block entry points, against the fp64 oracle.

A prompt P0 is shared by every path; a branch prefix B (tokens of its own, with their own loss)
is shared by two responses R1 and R2 (multi-level prefix trees, the adjacent workload the LongStraw
study notes cite beside branch replay). Replay composes from the library's calls:

* B is replayed once as a response against P0; its key gradients go into the fp32 accumulator
  rows of B (a block with q0 = 0).
* Each R_i is a block of the sequence [B; R_i]: its rows start at q0 = |B| and see B's keys and
  its own causally, so the block call adds its share of B's key gradients into the same rows.
  The caller places R_i's keys after B's (a copy into one slot) and reads R_i's own key
  gradients from the slot after the call.

The oracle replays B against P0, then each R_i against the prompt [P0; B]; the prompt-side
gradients are split back into P0's and B's parts and summed over the tree."""
import numpy as np
import pytest

from oracle import attn
from prefix_shared_branch_amd import inputs
from tests.helpers import check_bf16_out, check_fp32_accum, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,P,nb,children", [(64, 500, 70, (40, 55)), (128, 2000, 129, (64, 1))])
def test_two_level_prefix_tree(D, P, nb, children):
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=8, Hkv=2, Dqk=D, Dv=D, P=P, seed=71)
    f64 = inputs.bf16_bits_to_f64
    lens = [nb, *children]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    bits = {n: fn(cfg, 0, T) for n, fn in (("q", inputs.suffix_q), ("k", inputs.suffix_k), ("v", inputs.suffix_v),
                                           ("do", inputs.suffix_do))}
    kp_b, vp_b = inputs.prompt_k(cfg), inputs.prompt_v(cfg)
    dev = {n: dev_bf16(b) for n, b in bits.items()}
    kp, vp = dev_bf16(kp_b), dev_bf16(vp_b)
    Hkv = cfg.Hkv
    dkp = torch.zeros(P, Hkv, D, dtype=torch.float32, device="cuda")
    dvp = torch.zeros_like(dkp)
    rmax = max(children)
    # accumulator rows: B's (kept across calls), then one slot for the current child
    acc_k = torch.zeros(nb + rmax, Hkv, D, dtype=torch.float32, device="cuda")
    acc_v = torch.zeros_like(acc_k)
    slot_k = torch.empty(nb + rmax, Hkv, D, dtype=torch.bfloat16, device="cuda")
    slot_v = torch.empty_like(slot_k)
    slot_k[:nb] = dev["k"][:nb]
    slot_v[:nb] = dev["v"][:nb]
    got = {}
    # the branch, once, against the prompt
    sb = slice(0, nb)
    lo = torch.empty(max(nb, rmax), cfg.Hq, D, dtype=torch.bfloat16, device="cuda")   # O's rounding residual
    ob, lb = L.ls_replay_attn_fwd_block(dev["q"][sb], slot_k[:nb], slot_v[:nb], kp, vp, 0, cfg.scale, o_lo=lo[:nb])
    got["dQ_B"] = L.ls_replay_attn_bwd_block(dev["q"][sb], slot_k[:nb], slot_v[:nb], kp, vp, 0, ob, lb, dev["do"][sb],
                                             acc_k[:nb], acc_v[:nb], dkp, dvp, cfg.scale, o_lo=lo[:nb])
    got["O_B"], got["LSE_B"] = ob, lb
    for c, r in enumerate(children):
        s = slice(int(cu[1 + c]), int(cu[2 + c]))
        slot_k[nb:nb + r] = dev["k"][s]
        slot_v[nb:nb + r] = dev["v"][s]
        acc_k[nb:].zero_()
        acc_v[nb:].zero_()
        o, lse = L.ls_replay_attn_fwd_block(dev["q"][s], slot_k[:nb + r], slot_v[:nb + r], kp, vp, nb, cfg.scale,
                                            o_lo=lo[:r])
        dq = L.ls_replay_attn_bwd_block(dev["q"][s], slot_k[:nb + r], slot_v[:nb + r], kp, vp, nb, o, lse,
                                        dev["do"][s], acc_k[:nb + r], acc_v[:nb + r], dkp, dvp, cfg.scale,
                                        o_lo=lo[:r])
        got[f"O_{c}"], got[f"LSE_{c}"], got[f"dQ_{c}"] = o, lse, dq
        got[f"dK_{c}"], got[f"dV_{c}"] = acc_k[nb:nb + r].clone(), acc_v[nb:nb + r].clone()
    torch.cuda.synchronize()

    # oracle: B against P0, then each child against the prompt [P0; B]
    h = {n: f64(b) for n, b in bits.items()}
    Kp, Vp = f64(kp_b), f64(vp_b)
    dKp, dVp = np.zeros(Kp.shape), np.zeros(Vp.shape)
    B = slice(0, nb)
    O, LSE = attn.replay_attn_fwd(Kp, Vp, h["q"][B], h["k"][B], h["v"][B], [0, nb], cfg.scale)
    dQ, dKB, dVB = attn.replay_attn_bwd(Kp, Vp, h["q"][B], h["k"][B], h["v"][B], h["do"][B], [0, nb], cfg.scale,
                                        dKp, dVp)
    check_bf16_out(host_f64(got["O_B"]), O, "O_B")
    assert np.max(np.abs(host_f64(got["LSE_B"]) - LSE)) <= 1e-4
    check_bf16_out(host_f64(got["dQ_B"]), dQ, "dQ_B")
    Kpb, Vpb = np.concatenate([Kp, h["k"][B]]), np.concatenate([Vp, h["v"][B]])
    for c, r in enumerate(children):
        s = slice(int(cu[1 + c]), int(cu[2 + c]))
        acc = np.zeros(Kpb.shape), np.zeros(Vpb.shape)
        O, LSE = attn.replay_attn_fwd(Kpb, Vpb, h["q"][s], h["k"][s], h["v"][s], [0, r], cfg.scale)
        dQ, dKs, dVs = attn.replay_attn_bwd(Kpb, Vpb, h["q"][s], h["k"][s], h["v"][s], h["do"][s], [0, r], cfg.scale,
                                            *acc)
        dKp += acc[0][:P]
        dVp += acc[1][:P]
        dKB += acc[0][P:]
        dVB += acc[1][P:]
        check_bf16_out(host_f64(got[f"O_{c}"]), O, f"O_{c}")
        assert np.max(np.abs(host_f64(got[f"LSE_{c}"]) - LSE)) <= 1e-4
        check_bf16_out(host_f64(got[f"dQ_{c}"]), dQ, f"dQ_{c}")
        check_bf16_out(host_f64(got[f"dK_{c}"]), dKs, f"dK_{c}")
        check_bf16_out(host_f64(got[f"dV_{c}"]), dVs, f"dV_{c}")
    check_fp32_accum(host_f64(dkp), dKp, "dKp")
    check_fp32_accum(host_f64(dvp), dVp, "dVp")
    # the branch's key gradients: its own rows plus both children's (the block bar, as for any
    # response-key gradient kept in fp32)
    check_bf16_out(host_f64(acc_k[:nb]), dKB, "dK_B")
    check_bf16_out(host_f64(acc_v[:nb]), dVB, "dV_B")
