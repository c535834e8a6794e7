"""Central finite differences, float64.  TEST INFRASTRUCTURE ONLY.

Used to pin the analytic gradients of `attn` and `grpo` on micro shapes.
"""
from __future__ import annotations

import numpy as np


def grad(f, x, h=1e-6):
    """d f / d x for a scalar function f of the array x, by (f(x+h e) - f(x-h e)) / 2h per entry."""
    x = np.array(x, dtype=np.float64)
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for n in range(flat.size):
        keep = flat[n]
        flat[n] = keep + h
        fp = f(x)
        flat[n] = keep - h
        fm = f(x)
        flat[n] = keep
        gf[n] = (fp - fm) / (2 * h)
    return g
