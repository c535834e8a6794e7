"""Benchmark of the branch-replay hot path on one MI355X.

One step = one GRPO group of the named workload, replayed serially as the LongStraw study
notes prescribe (§2-1 step 4, §3-2 (4)): zero the resident prompt-gradient accumulators,
then for each of the G responses run replay attention forward, the fused clipped-GRPO token
loss over that response's logits, and replay attention backward (which adds the response's
prompt-side gradient in place). Inputs are seeded synthetic tensors already resident in HBM
when the timed region starts.

Prints one JSON line (rank 0). `value` = replayed response tokens per second of whole steps.
Also reported: the dominant kernel against its roofline, per-call times, algorithmic and
executed TFLOP/s, the loss kernel's GB/s, and the CPU oracle timed on a bounded sample.

usage: python bench.py [--steps K] [--warmup W] [--workload million] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from prefix_shared_branch_amd import inputs  # noqa: E402

METRIC = "replayed response tokens/s (fwd+bwd) at prompt P; % bf16 MFMA peak; loss GB/s"
PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s (at the 2.4 GHz peak clock)
PEAK_HBM = 8.0e12       # MI355X HBM3E, B/s
PEAK_CLOCK_GHZ = 2.4
# Shader clock the chip holds under these MFMA-dense kernels: SQ_BUSY_CYCLES over the dispatch time
# in the SQ counter runs of the attention kernels (1.68-1.77 GHz measured); the MFMA pipes peak at
# PEAK_BF16 * SUSTAINED_CLOCK_GHZ / PEAK_CLOCK_GHZ at that clock.
SUSTAINED_CLOCK_GHZ = 1.75


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="million", choices=["tiny", "mid", "long", "million", "mla"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle sample rows (0 = automatic)")
    ap.add_argument("--no-memory-receipt", action="store_true",
                    help="skip the peak-memory receipt (G = 2 vs G = 8 at mid, G = 2 vs G = 16 at million)")
    ap.add_argument("--memory-receipt-only", action="store_true", help="only run the peak-memory receipt")
    ap.add_argument("--no-receipts", action="store_true",
                    help="skip the attention receipts of the other workloads (Mid, Long, latent KV)")
    ap.add_argument("--receipts-only", action="store_true", help="only run the attention receipts")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of known size (HBM counter calibration)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Workload:
    """Resident inputs and reusable outputs/workspaces of one group."""

    def __init__(self, cfg):
        import torch
        from prefix_shared_branch_amd import lsreplay as L
        self.cfg = cfg
        self.R = inputs.response_lengths(cfg)
        self.G = int(cfg.G)
        self.cu = inputs.cu_seqlens(self.R)
        self.rewards = inputs.rewards(cfg)
        T = int(self.cu[-1])
        t0 = time.time()
        self.kp = to_dev(inputs.prompt_k(cfg))
        # latent KV: V is the leading Dv dims of the K rows (a strided view, no copy)
        self.vp = self.kp[:, :, :cfg.Dv] if cfg.mla else to_dev(inputs.prompt_v(cfg))
        log(f"prompt K/V resident ({(self.kp.numel() + (0 if cfg.mla else self.vp.numel())) * 2 / 2**30:.2f} GiB) "
            f"in {time.time() - t0:.1f}s")
        self.q = to_dev(inputs.suffix_q(cfg, 0, T))
        self.ks = to_dev(inputs.suffix_k(cfg, 0, T))
        self.vs = self.ks[:, :, :cfg.Dv] if cfg.mla else to_dev(inputs.suffix_v(cfg, 0, T))
        self.do = to_dev(inputs.suffix_do(cfg, 0, T))
        self.logits, self.targets, self.old = [], [], []
        t0 = time.time()
        for i in range(self.G):
            lg = to_dev(inputs.logits(cfg, i, 0, int(self.R[i])))
            y = torch.from_numpy(inputs.targets(cfg, i, int(self.R[i]))).cuda()
            # old-policy log-probs = current log-probs + N(0, sigma^2) noise (input synthesis only)
            lp = torch.empty(int(self.R[i]), dtype=torch.float32, device="cuda")
            for r0 in range(0, int(self.R[i]), 512):
                blk = lg[r0:r0 + 512].float()
                lp[r0:r0 + 512] = torch.log_softmax(blk, dim=1).gather(1, y[r0:r0 + 512, None].long())[:, 0]
                del blk
            noise = torch.from_numpy(inputs.old_logp_noise(cfg, i, int(self.R[i]))).cuda()
            self.logits.append(lg)
            self.targets.append(y)
            self.old.append(lp + noise)
            log(f"response {i}: logits [{int(self.R[i])}, {cfg.V}] resident")
        log(f"logits of {self.G} responses resident in {time.time() - t0:.1f}s")
        Rmax = int(self.R.max())
        dev = "cuda"
        self.dkp = torch.zeros(cfg.P, cfg.Hkv, cfg.Dqk, dtype=torch.float32, device=dev)
        self.dvp = torch.zeros(cfg.P, cfg.Hkv, cfg.Dv, dtype=torch.float32, device=dev)
        self.o = torch.empty(Rmax, cfg.Hq, cfg.Dv, dtype=torch.bfloat16, device=dev)
        self.o_lo = torch.empty(Rmax, cfg.Hq, cfg.Dv, dtype=torch.bfloat16, device=dev)  # O's rounding residual
        self.dq = torch.empty(Rmax, cfg.Hq, cfg.Dqk, dtype=torch.bfloat16, device=dev)
        self.dks = torch.empty(Rmax, cfg.Hkv, cfg.Dqk, dtype=torch.bfloat16, device=dev)
        self.dvs = torch.empty(Rmax, cfg.Hkv, cfg.Dv, dtype=torch.bfloat16, device=dev)
        self.dlogits = torch.empty(Rmax, cfg.V, dtype=torch.bfloat16, device=dev)
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        desc = L.make_desc(self.q, self.kp, self.vp, self.ks, self.vs, cfg.scale)
        wf = max(L.ls_replay_attn_workspace_bytes(desc, [0, int(r)], 0) for r in self.R)
        wb = max(L.ls_replay_attn_workspace_bytes(desc, [0, int(r)], 1) for r in self.R)
        wl = L.ls_grpo_workspace_bytes(Rmax, cfg.V)
        self.ws = torch.empty(max(wf, wb, wl, 256), dtype=torch.uint8, device=dev)
        self.lse = [torch.empty(cfg.Hq, int(r), dtype=torch.float32, device=dev) for r in self.R]

    def response(self, i, times=None, exact=True):
        import torch
        from prefix_shared_branch_amd import lsreplay as L
        cfg = self.cfg
        r0, r1 = int(self.cu[i]), int(self.cu[i + 1])
        R = r1 - r0
        sl = slice(r0, r1)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if times is not None else None
        if ev:
            ev[0].record()
        o, lse = L.ls_replay_attn_fwd(self.q[sl], self.ks[sl], self.vs[sl], self.kp, self.vp, [0, R], cfg.scale,
                                      out=self.o[:R], lse=self.lse[i], workspace=self.ws, o_lo=self.o_lo[:R])
        if ev:
            ev[1].record()
        L.ls_grpo_token_loss(self.logits[i], self.targets[i], self.old[i], self.R, self.rewards, cfg.eps, i, 1,
                             self.loss, dlogits=self.dlogits[:R], workspace=self.ws)
        if ev:
            ev[2].record()
        L.ls_replay_attn_bwd(self.q[sl], self.ks[sl], self.vs[sl], self.kp, self.vp, [0, R], o, lse, self.do[sl],
                             self.dkp if exact else None, self.dvp if exact else None, cfg.scale,
                             dq=self.dq[:R], dks=self.dks[:R], dvs=self.dvs[:R], workspace=self.ws, o_lo=self.o_lo[:R])
        if ev:
            ev[3].record()
            times.append(ev)

    def step(self, times=None):
        self.dkp.zero_()
        self.dvp.zero_()
        self.loss.zero_()
        for i in range(self.G):
            self.response(i, times)


def attn_receipt(cfg, n_resp):
    """Attention throughput of another workload: forward + backward with exact prompt gradients for
    its first n_resp responses, serially, after one untimed warm-up call on response 0. Each
    response's inputs are generated before its calls, outside the timed calls (no logits: the loss is
    measured by the main line)."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    kp = to_dev(inputs.prompt_k(cfg))
    vp = kp[:, :, :cfg.Dv] if cfg.mla else to_dev(inputs.prompt_v(cfg))
    dkp = torch.zeros(cfg.P, cfg.Hkv, cfg.Dqk, dtype=torch.float32, device="cuda")
    dvp = torch.zeros(cfg.P, cfg.Hkv, cfg.Dv, dtype=torch.float32, device="cuda")
    R = inputs.response_lengths(cfg)[:n_resp]
    cu = inputs.cu_seqlens(inputs.response_lengths(cfg))
    t_fwd = t_bwd = 0.0
    alg = 0
    for k in range(-1, n_resp):
        i = max(k, 0)
        r, t0 = int(R[i]), int(cu[i])
        q = to_dev(inputs.suffix_q(cfg, t0, t0 + r))
        ks = to_dev(inputs.suffix_k(cfg, t0, t0 + r))
        vs = ks[:, :, :cfg.Dv] if cfg.mla else to_dev(inputs.suffix_v(cfg, t0, t0 + r))
        do = to_dev(inputs.suffix_do(cfg, t0, t0 + r))
        lo = torch.empty(r, cfg.Hq, cfg.Dv, dtype=torch.bfloat16, device="cuda")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        o, lse = L.ls_replay_attn_fwd(q, ks, vs, kp, vp, [0, r], cfg.scale, o_lo=lo)
        ev[1].record()
        L.ls_replay_attn_bwd(q, ks, vs, kp, vp, [0, r], o, lse, do, dkp, dvp, cfg.scale, o_lo=lo)
        ev[2].record()
        torch.cuda.synchronize()
        if k >= 0:
            t_fwd += ev[0].elapsed_time(ev[1])
            t_bwd += ev[1].elapsed_time(ev[2])
            alg += flops(cfg, r)[0]
        del q, ks, vs, do, lo, o, lse
    tokens = int(R.sum())
    t = (t_fwd + t_bwd) * 1e-3
    out = {"workload": cfg.name, "P": cfg.P, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "Dqk": cfg.Dqk, "Dv": cfg.Dv,
           "responses": [int(x) for x in R], "tokens_per_s": tokens / t, "alg_TFLOPs": alg / t / 1e12,
           "alg_frac_peak": alg / t / PEAK_BF16, "fwd_ms": t_fwd, "bwd_ms": t_bwd}
    log(f"attention receipt {cfg.name}: {out['tokens_per_s']:.0f} tok/s, {out['alg_TFLOPs']:.0f} TFLOP/s")
    del kp, vp, dkp, dvp
    torch.cuda.empty_cache()
    return out


def receipts():
    """Attention receipts of the other named workloads: Mid (all 8 responses), Long (its first two
    responses as drawn, 2,461 and 2,414 tokens) and the latent-KV config at P = 262,144 (two
    responses of 4,096 tokens)."""
    mla = inputs.replace(inputs.CONFIGS["mla"], name="mla_p262k", P=262144, G=2, R_lo=4096, R_hi=4096)
    return [attn_receipt(inputs.CONFIGS["mid"], 8), attn_receipt(inputs.CONFIGS["long"], 2), attn_receipt(mla, 2)]


def memory_receipt(cfg, group_sizes):
    """Peak device memory of serial replay with each response's buffers alive only during its own
    replay (the response lifetime of the LongStraw study notes, §1-1 lifetime table and §2-1: the
    live graph is bounded by the current suffix). Per group size G: zero the resident accumulators,
    then for each of the G responses create its inputs (queries, suffix K/V, output gradient, logits,
    targets, old log-probs), its outputs and workspaces, run forward, loss and backward, and free
    them all. Resident across the group: prompt K/V and the fp32 prompt-gradient accumulators. The
    peak should not grow with G."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    kp = to_dev(inputs.prompt_k(cfg))
    vp = kp[:, :, :cfg.Dv] if cfg.mla else to_dev(inputs.prompt_v(cfg))
    dkp = torch.zeros(cfg.P, cfg.Hkv, cfg.Dqk, dtype=torch.float32, device="cuda")
    dvp = torch.zeros(cfg.P, cfg.Hkv, cfg.Dv, dtype=torch.float32, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    R_all = inputs.response_lengths(cfg)
    resident = torch.cuda.memory_allocated()
    out = {"workload": cfg.name, "resident_GiB": resident / 2**30, "peak_GiB": {}, "response_buffers_GiB": {}}
    for G in group_sizes:
        R = R_all[:G]
        rewards = inputs.rewards(cfg)[:G]
        cu = inputs.cu_seqlens(R_all)
        dkp.zero_()
        dvp.zero_()
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        biggest = 0
        for i in range(G):
            r = int(R[i])
            t0 = int(cu[i])
            q = to_dev(inputs.suffix_q(cfg, t0, t0 + r))
            ks = to_dev(inputs.suffix_k(cfg, t0, t0 + r))
            vs = ks[:, :, :cfg.Dv] if cfg.mla else to_dev(inputs.suffix_v(cfg, t0, t0 + r))
            do = to_dev(inputs.suffix_do(cfg, t0, t0 + r))
            lg = to_dev(inputs.logits(cfg, i, 0, r))
            y = torch.from_numpy(inputs.targets(cfg, i, r)).cuda()
            old = torch.from_numpy(inputs.old_logp_noise(cfg, i, r)).cuda()
            for r0 in range(0, r, 256):   # old = current log-probs + noise (input synthesis)
                old[r0:r0 + 256] += torch.log_softmax(lg[r0:r0 + 256].float(), dim=1).gather(
                    1, y[r0:r0 + 256, None].long())[:, 0]
            lo = torch.empty(r, cfg.Hq, cfg.Dv, dtype=torch.bfloat16, device="cuda")
            o, lse = L.ls_replay_attn_fwd(q, ks, vs, kp, vp, [0, r], cfg.scale, o_lo=lo)
            dl = L.ls_grpo_token_loss(lg, y, old, R, rewards, cfg.eps, i, 1, loss)
            L.ls_replay_attn_bwd(q, ks, vs, kp, vp, [0, r], o, lse, do, dkp, dvp, cfg.scale, o_lo=lo)
            torch.cuda.synchronize()
            biggest = max(biggest, torch.cuda.memory_allocated() - resident)
            del q, ks, vs, do, lg, y, old, lo, o, lse, dl
        torch.cuda.synchronize()
        out["peak_GiB"][str(G)] = torch.cuda.max_memory_allocated() / 2**30
        out["response_buffers_GiB"][str(G)] = biggest / 2**30
        log(f"memory receipt {cfg.name}: G={G} peak {out['peak_GiB'][str(G)]:.3f} GiB")
    gs = [str(g) for g in group_sizes]
    out["peak_delta_GiB"] = out["peak_GiB"][gs[-1]] - out["peak_GiB"][gs[0]]
    del kp, vp, dkp, dvp, loss
    torch.cuda.empty_cache()
    return out


def flops(cfg, R):
    """Algorithmic and executed MFMA flops of one response (per visible pair and query head)."""
    pairs = R * cfg.P + R * (R + 1) // 2
    d, dv = cfg.Dqk, cfg.Dv
    alg = 6 * (d + dv) * pairs * cfg.Hq
    # each product runs once (the dV / dK products in single-pass fp16): 1.5x the algorithmic work
    # at d = dv (2304 flops per pair-head at D = 128)
    executed = (2 * (d + dv) * pairs             # forward: S, PV
                + (2 * d + 2 * dv) * pairs       # dK/dV kernel: S, dP recomputed
                + (2 * dv + 2 * d) * pairs       # dK/dV kernel: dV, dK
                + (4 * d + 2 * dv) * pairs) * cfg.Hq   # dQ kernel: S, dP, dQ
    return alg, executed, pairs


def lmhead_measure(cfg, wl):
    """One call of the fused LM-head loss over response 0 (hidden size Hq * Dqk), timed after a warm-up
    call; also the scoring-only call (logits GEMM and loss, no gradient GEMMs)."""
    import torch
    from prefix_shared_branch_amd import lsreplay as L
    d = cfg.Hq * cfg.Dqk
    R0 = int(wl.R[0])
    H = to_dev(inputs.hidden(cfg, 0, 0, R0, d))
    W = to_dev(inputs.projection(cfg, d))
    dW = torch.zeros(cfg.V, d, dtype=torch.float32, device="cuda")
    dH = torch.empty(R0, d, dtype=torch.bfloat16, device="cuda")
    loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(L.ls_grpo_lmhead_workspace_bytes(R0, cfg.V, d), dtype=torch.uint8, device="cuda")
    args = (H, W, wl.targets[0], wl.old[0], wl.R, wl.rewards, cfg.eps, 0, 1, loss)
    L.ls_grpo_lmhead_loss(*args, dW_accum=dW, dH=dH, workspace=ws)     # warm-up (library handle, kernels)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    L.ls_grpo_lmhead_loss(*args, dW_accum=dW, dH=dH, workspace=ws)
    ev[1].record()
    L.ls_grpo_lmhead_loss(*args, workspace=ws, scoring_only=True)
    ev[2].record()
    torch.cuda.synchronize()
    t, ts = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    fl = 2.0 * R0 * cfg.V * d
    out = {"tokens": R0, "d": d, "vocab": cfg.V, "ms": t, "TFLOPs": 3 * fl / (t * 1e-3) / 1e12,
           "frac_peak": 3 * fl / (t * 1e-3) / PEAK_BF16, "scoring_ms": ts,
           "scoring_TFLOPs": fl / (ts * 1e-3) / 1e12}
    del H, W, dW, dH, ws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, rows):
    """Time the fp64 oracle on a bounded sample: the first `rows` rows of response 0 against the full
    prompt (an exact sub-problem), for the query heads of kv head 0, forward + backward with
    prompt-gradient accumulation; scaled to all kv heads (heads are independent). Plus the loss on
    256 rows of the vocabulary."""
    from oracle import attn, grpo
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    f64 = inputs.bf16_bits_to_f64
    g = cfg.Hq // cfg.Hkv
    Kp = f64(inputs.prompt_k(cfg)[:, :1, :])
    Vp = f64(inputs.prompt_v(cfg)[:, :1, :])
    Q = f64(inputs.suffix_q(cfg, 0, rows)[:, :g, :])
    Ks = f64(inputs.suffix_k(cfg, 0, rows)[:, :1, :])
    Vs = f64(inputs.suffix_v(cfg, 0, rows)[:, :1, :])
    dO = f64(inputs.suffix_do(cfg, 0, rows)[:, :g, :])
    dKp, dVp = np.zeros_like(Kp), np.zeros_like(Vp)
    t0 = time.time()
    attn.replay_attn_fwd(Kp, Vp, Q, Ks, Vs, [0, rows], cfg.scale)
    attn.replay_attn_bwd(Kp, Vp, Q, Ks, Vs, dO, [0, rows], cfg.scale, dKp, dVp)
    t_attn = time.time() - t0
    del Kp, Vp, dKp, dVp
    R = inputs.response_lengths(cfg)
    n = min(256, int(R[0]))
    x = f64(inputs.logits(cfg, 0, 0, n))
    y = inputs.targets(cfg, 0, n)
    old = grpo.token_logp(x, y) + inputs.old_logp_noise(cfg, 0, n)
    t0 = time.time()
    grpo.grpo_token_loss(x, y, old, np.concatenate([[n], R[1:]]), inputs.rewards(cfg), cfg.G, cfg.eps, 0, 1)
    t_loss = time.time() - t0
    loss_bytes = n * (4 * cfg.V + 12)
    return {"value": rows / (t_attn * cfg.Hkv), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 numpy oracle, first {rows} rows of response 0 against the full prompt P={cfg.P} "
                      f"(exact sub-problem), the {g} query heads of kv head 0, forward + backward with prompt-"
                      f"gradient accumulation: {t_attn:.1f}s, scaled by Hkv={cfg.Hkv}; loss on {n} rows of "
                      f"V={cfg.V}: {loss_bytes / t_loss / 1e9:.3f} GB/s",
            "loss_GBps": loss_bytes / t_loss / 1e9}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"replay_bwd_dkdv_prompt": ["replay_attn_dkdv64.hip", "common.h", "kernels.h"]}


def source_digest(kernel):
    """sha256 over the sources a kernel is compiled from (recorded counters are void once they change)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "prefix_shared_branch_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the recorded FETCH_SIZE / WRITE_SIZE counter runs, each scaled by
    the factor the same counter gave for a plain copy of known size; None if no record matches this
    kernel source and workload."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(kernel, {}).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != source_digest(kernel):
        return None
    return (rec["fetch_kib_per_launch"] * 1024 * rec["fetch_scale"]
            + rec["write_kib_per_launch"] * 1024 * rec["write_scale"])


def device_copy_GBps(n=1 << 30):
    """Bytes read + written per second by a plain device-to-device copy of n bytes (one warm-up, three
    timed): the HBM rate a simple streaming kernel reaches on this part, beside the 8 TB/s nameplate."""
    import torch
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    e0.record()
    for _ in range(3):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 3 * 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9


def copy_calibration():
    """A plain device copy of known size, for reading FETCH_SIZE / WRITE_SIZE against known bytes."""
    n = 1 << 30
    gbps = device_copy_GBps(n)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 4, "copy_GBps": gbps}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (the prompt-axis sharding "
              "design is documented, not built). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        torch.cuda.set_device(0)
        copy_calibration()
        return
    from prefix_shared_branch_amd import lsreplay as L
    L.lib()   # fail loudly if the HIP library is missing
    cfg = inputs.CONFIGS[args.workload]
    torch.cuda.set_device(0)
    if args.receipts_only:
        print(json.dumps(receipts()), flush=True)
        return
    if args.memory_receipt_only:
        print(json.dumps([memory_receipt(inputs.CONFIGS["mid"], [2, 8]),
                          memory_receipt(inputs.CONFIGS["million"], [2, 16])]), flush=True)
        return
    wl = Workload(cfg)
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    log("warmup done")

    times = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    L.ls_kernel_timer_start(L.LS_KERNEL_DKDV_PROMPT)
    e0.record()
    for _ in range(args.steps):
        wl.step(times)
    e1.record()
    torch.cuda.synchronize()
    dk_total, dk_launches = L.ls_kernel_timer_stop()
    wall = time.perf_counter() - t_start
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.1f} ms/step (host wall {wall:.1f}s)")

    t_fwd = sum(ev[0].elapsed_time(ev[1]) for ev in times) / args.steps
    t_loss = sum(ev[1].elapsed_time(ev[2]) for ev in times) / args.steps
    t_bwd = sum(ev[2].elapsed_time(ev[3]) for ev in times) / args.steps
    tokens = int(wl.R.sum())
    alg = exe = 0
    for r in wl.R:
        a, e, _ = flops(cfg, int(r))
        alg += a
        exe += e
    loss_bytes = tokens * (4 * cfg.V + 12)

    # scoring pass of the loss (old / reference policy: log-probs and loss share, no dlogits),
    # timed after the steps over the same logits: 2V + 12 bytes per token
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev_s[0].record()
    for i in range(wl.G):
        L.ls_grpo_token_loss(wl.logits[i], wl.targets[i], wl.old[i], wl.R, wl.rewards, cfg.eps, i, 1, wl.loss,
                             workspace=wl.ws, scoring_only=True)
    ev_s[1].record()
    torch.cuda.synchronize()
    t_score = ev_s[0].elapsed_time(ev_s[1])
    score_bytes = tokens * (2 * cfg.V + 12)

    # LM head fused with the loss (the step to the left of the loss) on the first response: hidden
    # size d = Hq * Dqk, logits = H W^T chunk by chunk; 3 GEMMs of 2 R V d flops each
    lm = lmhead_measure(cfg, wl)
    copy_gbps = device_copy_GBps()

    # dominant kernel: the dK/dV prompt kernel, timed by the library's kernel timer (HIP events on
    # the launch stream around every launch in the timed region)
    dkdv_ms = dk_total / max(1, dk_launches)
    dkdv_alg = sum(2 * (cfg.Dqk + cfg.Dv) * int(r) * cfg.P * cfg.Hq for r in wl.R) * args.steps / max(1, dk_launches)
    roof_ach = dkdv_alg / (dkdv_ms * 1e-3) / 1e12
    traffic = recorded_traffic("replay_bwd_dkdv_prompt", cfg.name)
    fwd_alg = sum(2 * (cfg.Dqk + cfg.Dv) * flops(cfg, int(r))[2] * cfg.Hq for r in wl.R)   # per group

    out = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "P": cfg.P, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "Dqk": cfg.Dqk, "Dv": cfg.Dv,
                   "G": cfg.G, "R": [int(r) for r in wl.R] if len(set(wl.R.tolist())) > 1 else int(wl.R[0]),
                   "vocab": cfg.V, "eps": cfg.eps, "gradient_semantics": "exact-prompt-grad"},
        "roofline": {"bound": "mfma", "achieved": roof_ach, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                     "frac": roof_ach / (PEAK_BF16 / 1e12), "traffic": traffic,
                     "kernel": "replay_bwd_dkdv_w64 (prompt keys)", "avg_ms": dkdv_ms, "launches": dk_launches,
                     "alg_flops_per_launch": dkdv_alg},
        "detail": {
            "attn_tokens_per_s": tokens / ((t_fwd + t_bwd) * 1e-3),
            "attn_alg_TFLOPs": alg / ((t_fwd + t_bwd) * 1e-3) / 1e12,
            "attn_alg_frac_peak": alg / ((t_fwd + t_bwd) * 1e-3) / PEAK_BF16,
            "attn_exec_TFLOPs": exe / ((t_fwd + t_bwd) * 1e-3) / 1e12,
            "attn_exec_over_alg": exe / alg,
            # executed rate over the MFMA peak at the sustained clock: an estimate of the share of
            # cycles the MFMA pipes are busy (the SQ counter runs measure it per kernel)
            "mfma_busy_est": exe / ((t_fwd + t_bwd) * 1e-3) / (PEAK_BF16 * SUSTAINED_CLOCK_GHZ / PEAK_CLOCK_GHZ),
            "sustained_clock_GHz": SUSTAINED_CLOCK_GHZ,
            "fwd_ms_per_group": t_fwd, "bwd_ms_per_group": t_bwd, "loss_ms_per_group": t_loss,
            "fwd_alg_TFLOPs": fwd_alg / (t_fwd * 1e-3) / 1e12,
            "loss_GBps": loss_bytes / (t_loss * 1e-3) / 1e9,
            "loss_frac_hbm": loss_bytes / (t_loss * 1e-3) / PEAK_HBM,
            "copy_GBps": copy_gbps,
            "loss_frac_copy": loss_bytes / (t_loss * 1e-3) / 1e9 / copy_gbps,
            "scoring_loss_ms_per_group": t_score,
            "scoring_loss_GBps": score_bytes / (t_score * 1e-3) / 1e9,
            "lmhead": lm,
            # the timed run keeps every response's logits resident (input generation stays out of the
            # timed region); memory_receipt below measures the per-response lifetime instead
            "peak_mem_GiB_timed_run": torch.cuda.max_memory_allocated() / 2**30,
            "pages_context": "2.1M token positions on eight H20 GPUs (whole model, end to end; not comparable)",
        },
    }
    del wl
    torch.cuda.empty_cache()
    if not args.no_receipts:
        out["detail"]["receipts"] = receipts()
    if not args.no_memory_receipt:
        # outside the timed region: each response's buffers live only during its own replay
        out["detail"]["memory_receipt"] = [memory_receipt(inputs.CONFIGS["mid"], [2, 8]),
                                           memory_receipt(inputs.CONFIGS["million"], [2, 16])]
    if not args.no_cpu_baseline:
        # about 10-30 s of oracle work: the sample shrinks as the prompt grows
        rows = args.cpu_rows or int(min(256, max(1, (1 << 25) // max(1, cfg.P))))
        log(f"cpu baseline: oracle on {rows} rows")
        out["cpu_baseline"] = cpu_baseline(cfg, rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
