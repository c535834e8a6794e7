"""Shared test utilities: device upload of generator outputs and the parity tolerances.

Tolerances (bf16 outputs: max-abs 2e-2 literally, plus scale-aware per-head norms; fp32
accumulators and the loss: 1e-3 relative) follow the parity bar for replay attention and the
GRPO objective; the scale-aware forms are needed because typical |O| at long prompts is far
below 2e-2 and normalised advantages make the loss itself close to zero.
"""
from __future__ import annotations

import numpy as np

from prefix_shared_branch_amd import inputs


def dev_bf16(bits: np.ndarray):
    """uint16 bf16 bit patterns -> CUDA bfloat16 tensor of the same shape (strides preserved if contiguous)."""
    import torch
    a = np.ascontiguousarray(bits)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return inputs.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().double().cpu().numpy()


def check_bf16_out(got, ref, name, head_axis=1, literal_abs=True):
    """Per head: ||d||_inf <= 2e-2 ||ref||_inf, ||d||_2 <= 1e-2 ||ref||_2; and (literal_abs) the
    stated overall max-abs <= 2e-2, which is meaningful where |ref| < 1 (the named workloads).
    Edge cases with |ref| of several units (one bf16 ulp at 4 is 0.03) rely on the relative forms."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = got - ref
    if literal_abs:
        assert np.max(np.abs(d), initial=0.0) <= 2e-2, f"{name}: max-abs {np.max(np.abs(d))}"
    for h in range(ref.shape[head_axis]):
        dh = np.take(d, h, axis=head_axis)
        rh = np.take(ref, h, axis=head_axis)
        rinf, r2 = np.max(np.abs(rh), initial=0.0), np.linalg.norm(rh)
        if r2 == 0:
            assert np.max(np.abs(dh), initial=0.0) == 0.0, f"{name} head {h}: ref zero, got nonzero"
            continue
        einf, e2 = np.max(np.abs(dh)) / rinf, np.linalg.norm(dh) / r2
        assert einf <= 2e-2 and e2 <= 1e-2, f"{name} head {h}: rel inf {einf:.3e}, rel l2 {e2:.3e}"


def check_fp32_accum(got, ref, name, head_axis=1, tol=1e-3, tol_inf=1e-2):
    """Per kv head: ||d||_2 <= tol ||ref||_2 and, element-wise, ||d||_inf <= tol_inf ||ref||_inf.

    The L2 form is the 1e-3 relative bar of the fp32 accumulators; the infinity form catches a
    localised error (one wrong key tile moves the L2 ratio of a long prompt very little). Prints the
    worst ratios of both forms and returns them."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    worst2 = worst_inf = 0.0
    for h in range(ref.shape[head_axis]):
        dh = np.take(got - ref, h, axis=head_axis)
        rh = np.take(ref, h, axis=head_axis)
        e2 = np.linalg.norm(dh) / max(np.linalg.norm(rh), 1e-300)
        einf = np.max(np.abs(dh), initial=0.0) / max(np.max(np.abs(rh), initial=0.0), 1e-300)
        worst2, worst_inf = max(worst2, e2), max(worst_inf, einf)
        assert e2 <= tol, f"{name} kv head {h}: rel l2 {e2:.3e} > {tol}"
        assert einf <= tol_inf, f"{name} kv head {h}: rel inf {einf:.3e} > {tol_inf}"
    print(f"[parity] {name}: rel l2 {worst2:.3e} (bar {tol}), rel inf {worst_inf:.3e} (bar {tol_inf})", flush=True)
    return worst2


def rel_l2(got, ref):
    return float(np.linalg.norm(np.asarray(got) - np.asarray(ref)) / max(np.linalg.norm(ref), 1e-300))
