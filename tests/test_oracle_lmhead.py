"""Pins of the LM-head + GRPO-loss oracle (CPU only).

Sources of truth: central finite differences of the loss in the hidden states and in the
projection (shapes with d != V, so a transposed operand fails them); the identity projection,
which reduces the composition to the pinned loss oracle; and bf16 rounding on hand-picked values
(ties to even at 1 + 2^-8 and 1 + 3*2^-8, one bf16 ulp at 1 being 2^-7).
"""
import numpy as np
import pytest

from oracle import fd, grpo, lmhead


def _case(seed, G=3, d=5, V=7, lo=2, hi=4):
    g = np.random.default_rng(seed)
    R = g.integers(lo, hi + 1, size=G)
    T = int(R.sum())
    H = g.standard_normal((T, d))
    W = g.standard_normal((V, d)) * 0.7
    y = g.integers(0, V, size=T)
    r = (g.random(G) < 0.5).astype(np.float64)
    if r.min() == r.max():
        r[0] = 1 - r[0]
    old = grpo.token_logp(H @ W.T, y) + g.standard_normal(T) * 0.4
    return R, H, W, y, r, old


def test_round_bf16_values():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -7, -2.5, 3.0e-3, 65504.0, 1 + 2.0 ** -8 + 2.0 ** -20])
    # 3e-3 = 1.536 * 2^-9 and 1.536 * 128 = 196.6, so the nearest bf16 is 197/128 * 2^-9; 65504 lies
    # past the last 8-bit significand below 2^16 (65280) by more than half a step, so it rounds up
    want = np.array([1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -2.5, 197 / 128 * 2.0 ** -9, 65536.0, 1 + 2.0 ** -7])
    np.testing.assert_array_equal(lmhead.round_bf16(x), want)


def test_finite_differences_in_hidden_and_projection():
    R, H, W, y, r, old = _case(1)
    G, eps = 3, 0.2
    loss, dH, dW, _, _ = lmhead.lmhead_grpo_loss(H, W, y, old, R, r, G, eps, 0, G, round_logits=False)
    fH = fd.grad(lambda z: lmhead.lmhead_grpo_loss(z, W, y, old, R, r, G, eps, 0, G, round_logits=False)[0], H, h=1e-6)
    fW = fd.grad(lambda z: lmhead.lmhead_grpo_loss(H, z, y, old, R, r, G, eps, 0, G, round_logits=False)[0], W, h=1e-6)
    assert np.max(np.abs(fH - dH)) < 1e-7 * max(1.0, np.max(np.abs(dH)))
    assert np.max(np.abs(fW - dW)) < 1e-7 * max(1.0, np.max(np.abs(dW)))
    assert np.abs(dH).max() > 1e-3 and np.abs(dW).max() > 1e-3   # the check is not vacuous


def test_identity_projection_reduces_to_loss_oracle():
    g = np.random.default_rng(2)
    R = np.array([3, 2])
    T, V = 5, 6
    H = g.standard_normal((T, V)) * 2
    y = g.integers(0, V, size=T)
    old = grpo.token_logp(H, y) + g.standard_normal(T) * 0.3
    r = np.array([1.0, 0.0])
    loss, dH, dW, logp, clip = lmhead.lmhead_grpo_loss(H, np.eye(V), y, old, R, r, 2, 0.2, 0, 2, round_logits=False)
    l2, dl, lp2, c2 = grpo.grpo_token_loss(H, y, old, R, r, 2, 0.2, 0, 2)
    assert loss == l2
    np.testing.assert_array_equal(dH, dl)
    np.testing.assert_allclose(dW, dl.T @ H, rtol=0, atol=0)
    np.testing.assert_array_equal(logp, lp2)
    np.testing.assert_array_equal(clip, c2)


def test_rounded_logits_feed_the_loss():
    """With rounding on, the loss equals the loss oracle on the rounded product."""
    R, H, W, y, r, old = _case(3, d=9, V=11)
    loss, dH, dW, logp, _ = lmhead.lmhead_grpo_loss(H, W, y, old, R, r, 3, 0.2, 0, 3)
    x = lmhead.round_bf16(H @ W.T)
    assert np.all(x != H @ W.T)          # the rounding is not the identity on these inputs
    l2, dl, lp2, _ = grpo.grpo_token_loss(x, y, old, R, r, 3, 0.2, 0, 3)
    assert loss == l2
    np.testing.assert_array_equal(logp, lp2)
    np.testing.assert_allclose(dH, dl @ W, rtol=1e-15, atol=0)
