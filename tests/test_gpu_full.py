"""GPU parity at the full prompt lengths of the long and Million-token workloads.

Replay attention at P = 262,144 and P = 1,048,576 (LongStraw study notes §2-1 step 4, §3-2 (2)/(4)).

* **Short responses.** The GPU runs every head of the configuration. The oracle recomputes the first
  and the last kv head and their query heads in full: O, LSE, dQ, dKs, dVs, and the prompt dK/dV
  accumulators element by element (the last kv head's accumulator rows sit at the highest
  addresses). Heads are independent, and a response's first rows form an exact sub-problem, since
  row t sees only suffix keys up to t. At the Million-token prompt 64 rows are checked: 320
  GQA-packed rows, ten 32-row steps of the dK/dV kernel's sweep, so its load ring turns over
  several times.
* **Full response.** Response 0 of the Million workload runs in the launch configuration the
  benchmark times: one call per 4,096-token response, with exact prompt gradients.
  * O, LSE and dQ are checked on sampled rows. Each row depends on that row alone.
  * The value-gradient column sums are checked for every kv head. For each kv head k,
    Σ_j dV_P[j,k] + Σ_s dVs[s,k] = Σ_t Σ_{h in k} dO[t,h], because each row's softmax weights sum
    to one. This holds at any size and needs no O(P·R) oracle work.
"""
import numpy as np
import pytest

from oracle import attn
from prefix_shared_branch_amd import inputs
from tests.helpers import check_bf16_out, check_fp32_accum, dev_bf16, host_f64

pytestmark = pytest.mark.gpu

f64 = inputs.bf16_bits_to_f64


class Prompt:
    """Full-size prompt K/V of a config: device copies (all heads) and float64 slices of the first
    and the last kv head."""

    def __init__(self, cfg):
        import torch
        self.cfg = cfg
        kp, vp = inputs.prompt_k(cfg), inputs.prompt_v(cfg)
        self.kp, self.vp = dev_bf16(kp), dev_bf16(vp)
        self.heads = sorted({0, cfg.Hkv - 1})
        self.kph = {k: f64(kp[:, k:k + 1, :]) for k in self.heads}
        self.vph = {k: f64(vp[:, k:k + 1, :]) for k in self.heads}
        self.kp0, self.vp0 = self.kph[0], self.vph[0]
        del kp, vp
        self.torch = torch

    def run(self, r, exact=True):
        """fwd + bwd of the first r rows of response 0 on the GPU (one call each)."""
        from prefix_shared_branch_amd import lsreplay as L
        t, cfg = self.torch, self.cfg
        bits = {n: fn(cfg, 0, r) for n, fn in (("q", inputs.suffix_q), ("ks", inputs.suffix_k),
                                                ("vs", inputs.suffix_v), ("do", inputs.suffix_do))}
        d = {n: dev_bf16(b) for n, b in bits.items()}
        dkp = t.zeros(cfg.P, cfg.Hkv, cfg.Dqk, dtype=t.float32, device="cuda") if exact else None
        dvp = t.zeros(cfg.P, cfg.Hkv, cfg.Dv, dtype=t.float32, device="cuda") if exact else None
        lo = t.empty(r, cfg.Hq, cfg.Dv, dtype=t.bfloat16, device="cuda")
        o, lse = L.ls_replay_attn_fwd(d["q"], d["ks"], d["vs"], self.kp, self.vp, [0, r], cfg.scale, o_lo=lo)
        dq, dks, dvs = L.ls_replay_attn_bwd(d["q"], d["ks"], d["vs"], self.kp, self.vp, [0, r], o, lse, d["do"],
                                            dkp, dvp, cfg.scale, o_lo=lo)
        t.cuda.synchronize()
        return bits, dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp)


def _head_operands(cfg, bits, k):
    """float64 operands of kv head k: its g query heads, its keys / values, their output gradients."""
    g = cfg.Hq // cfg.Hkv
    qs = slice(k * g, (k + 1) * g)
    return (f64(bits["q"][:, qs, :]), f64(bits["ks"][:, k:k + 1, :]), f64(bits["vs"][:, k:k + 1, :]),
            f64(bits["do"][:, qs, :]), g)


def _check_short(pr, r):
    cfg = pr.cfg
    bits, got = pr.run(r)
    cu = [0, r]
    for k in pr.heads:
        print(f"[parity] P={cfg.P} rows={r} kv head {k}", flush=True)
        Q, Ks, Vs, dO, g = _head_operands(cfg, bits, k)
        qs, ks = slice(k * g, (k + 1) * g), slice(k, k + 1)
        kp, vp = pr.kph[k], pr.vph[k]
        O, LSE = attn.replay_attn_fwd(kp, vp, Q, Ks, Vs, cu, cfg.scale)
        dKp, dVp = np.zeros(kp.shape), np.zeros(vp.shape)
        dQ, dKs, dVs = attn.replay_attn_bwd(kp, vp, Q, Ks, Vs, dO, cu, cfg.scale, dKp, dVp)
        check_bf16_out(host_f64(got["O"][:, qs]), O, "O")
        lse = host_f64(got["LSE"][qs])
        assert np.max(np.abs(lse - LSE)) <= 1e-4, np.max(np.abs(lse - LSE))
        check_bf16_out(host_f64(got["dQ"][:, qs]), dQ, "dQ")
        check_bf16_out(host_f64(got["dKs"][:, ks]), dKs, "dKs")
        check_bf16_out(host_f64(got["dVs"][:, ks]), dVs, "dVs")
        check_fp32_accum(host_f64(got["dKp"][:, ks]), dKp, f"dKp kv head {k}")
        check_fp32_accum(host_f64(got["dVp"][:, ks]), dVp, f"dVp kv head {k}")


def test_long_prompt_short_response():
    pr = Prompt(inputs.CONFIGS["long"])
    _check_short(pr, 40)


@pytest.fixture(scope="module")
def million():
    return Prompt(inputs.CONFIGS["million"])


def test_million_prompt_short_response(million):
    _check_short(million, 64)


def test_million_full_response_sampled_rows_and_column_sums(million):
    pr, cfg = million, million.cfg
    r = int(inputs.response_lengths(cfg)[0])
    bits, got = pr.run(r)
    Q, Ks, Vs, dO, g = _head_operands(cfg, bits, 0)
    rows = np.array([0, 63, 2047, r - 1])
    O, LSE = attn.replay_attn_fwd(pr.kp0, pr.vp0, Q, Ks, Vs, [0, r], cfg.scale, rows=rows)
    check_bf16_out(host_f64(got["O"][rows, :g]), O[rows], "O rows")
    lse = host_f64(got["LSE"][:g])[:, rows]
    d = lse - LSE[:, rows]
    assert np.max(np.abs(d)) <= 1e-4, f"LSE rows {rows.tolist()}: signed differences by head\n{d}"

    dQ = attn.replay_attn_bwd_rows(pr.kp0, pr.vp0, Q, Ks, Vs, dO, [0, r], cfg.scale, rows)
    check_bf16_out(host_f64(got["dQ"][rows, :g]), dQ, "dQ rows")

    # column sums of the value gradient, every kv head (fp32 sums of P + R terms)
    do_all = f64(bits["do"]).reshape(r, cfg.Hkv, g, cfg.Dv)
    want = do_all.sum(axis=(0, 2))                                       # [Hkv, Dv]
    have = (got["dVp"].double().sum(dim=0) + got["dVs"].double().sum(dim=0)).cpu().numpy()
    for k in range(cfg.Hkv):
        rel = np.linalg.norm(have[k] - want[k]) / np.linalg.norm(want[k])
        assert rel <= 1e-3, (k, rel)

    # Key-gradient identities, every kv head, over the prompt and the response keys. Each row's dS
    # sums to zero over its keys (its softmax weights sum to one and Delta = dO . O), so
    # sum_j dK_j = 0. And dK = scale dS^T Q with dQ = scale dS K gives dK^T K = Q^T dQ, summed over
    # the kv head's query heads. The first bounds the accumulated sums against their absolute sums
    # (each key's error enters alone, a wrong tile shows), the second fixes their scale.
    import torch
    Qd = dev_bf16(bits["q"]).double().reshape(r, cfg.Hkv, g, cfg.Dqk)
    dQd = got["dQ"].double().reshape(r, cfg.Hkv, g, cfg.Dqk)
    for k in range(cfg.Hkv):
        dkp = got["dKp"][:, k, :].double()
        dks = got["dKs"][:, k, :].double()
        tot = dkp.sum(dim=0) + dks.sum(dim=0)
        mag = dkp.abs().sum(dim=0) + dks.abs().sum(dim=0)
        e1 = float(torch.linalg.norm(tot) / torch.linalg.norm(mag))
        lhs = (dkp.T.contiguous() @ pr.kp[:, k, :].double().contiguous()
               + dks.T.contiguous() @ dev_bf16(bits["ks"][:, k, :]).double().contiguous())
        qk = Qd[:, k].reshape(r * g, cfg.Dqk)
        rhs = qk.T.contiguous() @ dQd[:, k].reshape(r * g, cfg.Dqk).contiguous()
        e2 = float(torch.linalg.norm(lhs - rhs) / torch.linalg.norm(rhs))
        print(f"[parity] kv head {k}: |sum dK| / sum |dK| = {e1:.2e}, dK^T K vs Q^T dQ rel {e2:.2e}", flush=True)
        assert e1 <= 1e-4, (k, e1)
        assert e2 <= 2e-2, (k, e2)
