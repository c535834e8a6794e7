"""Seeded synthetic inputs for replay attention and the clipped-GRPO token loss.

This module only draws random numbers and stores them: it computes nothing of the
method itself. Both the CPU oracle (through the tests) and the GPU path (through
the tests and the benchmark) take their inputs from here, so the two sides see
bit-identical bf16 values.

Every tensor is chunk-addressable: chunk c of tensor `tid` is drawn from
``numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=(tid, sub, c))))``,
so any slice of a multi-million-row prompt can be regenerated on its own, and
chunks can be drawn in parallel threads.

Workload shapes follow the LongStraw study notes (dimensionstp.github.io,
"LongStraw" summary): one shared prompt of length P, a group of G responses of
lengths R_i (§1-1 problem definition), binary rewards (§4-1 data).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids (part of the seed derivation; never renumber)
TID_Q, TID_KP, TID_VP, TID_KS, TID_VS, TID_DO = 1, 2, 3, 4, 5, 6
TID_LOGITS, TID_TARGETS, TID_OLD_NOISE, TID_REWARDS, TID_LENGTHS = 7, 8, 9, 10, 11
TID_HIDDEN, TID_PROJ = 12, 13

CHUNK_ELEMS = 1 << 22  # elements per generator chunk (rows are never split)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    Hq: int
    Hkv: int
    Dqk: int
    Dv: int
    P: int
    G: int
    R_lo: int
    R_hi: int
    attn_sigma: float      # std of Q, K, V, dO entries
    mla: bool              # V is the first Dv dims of the K buffer (latent KV)
    V: int                 # vocabulary size
    logit_sigma: float     # std of logits
    old_sigma: float       # std of the noise added to current log-probs to form old log-probs
    eps: float
    reward_p: float        # Bernoulli parameter of binary rewards
    seed: int

    @property
    def ldk(self) -> int:
        return self.Hkv * self.Dqk

    @property
    def ldv(self) -> int:
        # latent KV: V rows live inside the K rows (same row stride)
        return self.ldk if self.mla else self.Hkv * self.Dv

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.Dqk))


CONFIGS = {
    "tiny": Config("tiny", 8, 2, 64, 64, 1024, 4, 64, 128, 1.0, False, 4096, 2.0, 0.05, 0.2, 0.5, 1),
    "mid": Config("mid", 32, 8, 128, 128, 32768, 8, 1024, 1024, 1.0, False, 151936, 2.0, 0.05, 0.2, 0.5, 2),
    "long": Config("long", 24, 4, 128, 128, 262144, 8, 2048, 8192, 1.0, False, 151936, 2.0, 0.05, 0.2, 0.3, 3),
    "million": Config("million", 40, 8, 128, 128, 1048576, 16, 4096, 4096, 1.0, False, 151936, 2.0, 0.05, 0.2,
                      0.5, 4),
    "mla": Config("mla", 16, 1, 576, 512, 2097152, 8, 4096, 8192, 1.0 / 24.0, True, 151936, 2.0, 0.05, 0.2, 0.5, 5),
    # test-only variants
    "tiny_clip": Config("tiny_clip", 8, 2, 64, 64, 1024, 4, 64, 128, 1.0, False, 4096, 2.0, 0.25, 0.2, 0.5, 11),
    "micro": Config("micro", 2, 1, 4, 4, 6, 2, 3, 5, 1.0, False, 7, 2.0, 0.25, 0.2, 0.5, 21),
}


def replace(cfg: Config, **kw) -> Config:
    return dataclasses.replace(cfg, **kw)


# ---------------------------------------------------------------- bf16 storage
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------- generators
def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16_rows(seed: int, tid: int, sub: int, row0: int, row1: int, row_elems: int, sigma: float,
                     out: np.ndarray | None = None) -> np.ndarray:
    """Rows [row0, row1) of an N(0, sigma^2) tensor with `row_elems` entries per row, as bf16 bits.

    Row r is always drawn by chunk r // rows_per_chunk, so a slice equals the same rows of the whole tensor.
    """
    rpc = max(1, CHUNK_ELEMS // row_elems)
    n = row1 - row0
    if out is None:
        out = np.empty((n, row_elems), dtype=np.uint16)
    if n <= 0:
        return out
    c0, c1 = row0 // rpc, (row1 - 1) // rpc

    def work(c):
        cr0, cr1 = c * rpc, (c + 1) * rpc
        g = _rng(seed, tid, sub, c)
        lo, hi = max(cr0, row0), min(cr1, row1)
        # draw the whole chunk prefix up to `hi` so that a row's value never depends on the slice requested
        vals = g.standard_normal((hi - cr0) * row_elems, dtype=np.float32)[(lo - cr0) * row_elems:]
        vals *= np.float32(sigma)
        out[lo - row0:hi - row0] = f32_to_bf16_bits(vals).reshape(hi - lo, row_elems)

    chunks = range(c0, c1 + 1)
    if len(chunks) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, chunks))
    else:
        work(c0)
    return out


def response_lengths(cfg: Config) -> np.ndarray:
    """R_i, integers uniform in [R_lo, R_hi] inclusive."""
    g = _rng(cfg.seed, TID_LENGTHS)
    return g.integers(cfg.R_lo, cfg.R_hi + 1, size=cfg.G).astype(np.int32)


def cu_seqlens(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def rewards(cfg: Config) -> np.ndarray:
    """Binary rewards r_i ~ Bernoulli(p) in {0, 1}, float32."""
    g = _rng(cfg.seed, TID_REWARDS)
    return (g.random(cfg.G) < cfg.reward_p).astype(np.float32)


# ---- attention tensors. Layouts (row = token):
#   Kp [P, Hkv, Dqk] (MLA: [P, 1, Dqk], V = first Dv dims), Vp [P, Hkv, Dv]
#   Q [T, Hq, Dqk], Ks [T, Hkv, Dqk], Vs [T, Hkv, Dv], dO [T, Hq, Dv]   (T = sum of R_i, responses packed)
def prompt_k(cfg: Config, row0: int = 0, row1: int | None = None) -> np.ndarray:
    row1 = cfg.P if row1 is None else row1
    return normal_bf16_rows(cfg.seed, TID_KP, 0, row0, row1, cfg.Hkv * cfg.Dqk, cfg.attn_sigma).reshape(
        -1, cfg.Hkv, cfg.Dqk)


def prompt_v(cfg: Config, row0: int = 0, row1: int | None = None) -> np.ndarray:
    """Prompt V. For latent KV this is a strided view of the K rows (first Dv dims)."""
    if cfg.mla:
        return prompt_k(cfg, row0, row1)[:, :, :cfg.Dv]
    row1 = cfg.P if row1 is None else row1
    return normal_bf16_rows(cfg.seed, TID_VP, 0, row0, row1, cfg.Hkv * cfg.Dv, cfg.attn_sigma).reshape(
        -1, cfg.Hkv, cfg.Dv)


def suffix_q(cfg: Config, t0: int, t1: int) -> np.ndarray:
    return normal_bf16_rows(cfg.seed, TID_Q, 0, t0, t1, cfg.Hq * cfg.Dqk, cfg.attn_sigma).reshape(-1, cfg.Hq, cfg.Dqk)


def suffix_k(cfg: Config, t0: int, t1: int) -> np.ndarray:
    return normal_bf16_rows(cfg.seed, TID_KS, 0, t0, t1, cfg.Hkv * cfg.Dqk, cfg.attn_sigma).reshape(
        -1, cfg.Hkv, cfg.Dqk)


def suffix_v(cfg: Config, t0: int, t1: int) -> np.ndarray:
    if cfg.mla:
        return suffix_k(cfg, t0, t1)[:, :, :cfg.Dv]
    return normal_bf16_rows(cfg.seed, TID_VS, 0, t0, t1, cfg.Hkv * cfg.Dv, cfg.attn_sigma).reshape(-1, cfg.Hkv, cfg.Dv)


def suffix_do(cfg: Config, t0: int, t1: int) -> np.ndarray:
    return normal_bf16_rows(cfg.seed, TID_DO, 0, t0, t1, cfg.Hq * cfg.Dv, cfg.attn_sigma).reshape(-1, cfg.Hq, cfg.Dv)


# ---- loss tensors, per response i: logits [R_i, V] bf16, targets [R_i] int32, old-logp noise [R_i] fp32
def logits(cfg: Config, i: int, r0: int, r1: int) -> np.ndarray:
    return normal_bf16_rows(cfg.seed, TID_LOGITS, i, r0, r1, cfg.V, cfg.logit_sigma)


def targets(cfg: Config, i: int, n: int) -> np.ndarray:
    """Sampled token ids, uniform in [0, V)."""
    return _rng(cfg.seed, TID_TARGETS, i).integers(0, cfg.V, size=n).astype(np.int32)


def old_logp_noise(cfg: Config, i: int, n: int) -> np.ndarray:
    """N(0, old_sigma^2) noise; old-policy log-probs are the current log-probs plus this noise."""
    return (_rng(cfg.seed, TID_OLD_NOISE, i).standard_normal(n) * cfg.old_sigma).astype(np.float32)


# ---- LM-head tensors (LM head fused with the loss): hidden states H [R_i, d] ~ N(0, 1) per response i,
# and the vocabulary projection W [V, d] ~ N(0, (logit_sigma / sqrt(d))^2), so that the logits H W^T
# have about the loss configs' spread (standard deviation logit_sigma).
def hidden(cfg: Config, i: int, r0: int, r1: int, d: int) -> np.ndarray:
    return normal_bf16_rows(cfg.seed, TID_HIDDEN, i, r0, r1, d, 1.0)


def projection(cfg: Config, d: int) -> np.ndarray:
    return normal_bf16_rows(cfg.seed, TID_PROJ, 0, 0, cfg.V, d, cfg.logit_sigma / float(np.sqrt(d)))
