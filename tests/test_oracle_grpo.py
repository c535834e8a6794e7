"""Pins of the GRPO objective oracle (CPU only).

Sources of truth: closed forms of the clipped objective of the LongStraw study notes
(§1-1, L_policy equation) at rho = 1 and on clipped tokens, uniform logits,
scipy's log_softmax / softmax and torch float64 autograd (library routines), central
finite differences on a 7-word vocabulary, and properties of the group advantage.
"""
import numpy as np
import pytest
import scipy.special

from oracle import fd, grpo


def _case(seed, G=4, V=7, lo=2, hi=5, sigma=2.0):
    g = np.random.default_rng(seed)
    R = g.integers(lo, hi + 1, size=G)
    T = int(R.sum())
    x = g.standard_normal((T, V)) * sigma
    y = g.integers(0, V, size=T)
    r = (g.random(G) < 0.5).astype(np.float64)
    if r.min() == r.max():
        r[0] = 1 - r[0]
    return R, x, y, r


def test_logp_matches_scipy_and_uniform():
    R, x, y, r = _case(1, V=11)
    lp = grpo.token_logp(x, y)
    ref = scipy.special.log_softmax(x, axis=1)[np.arange(x.shape[0]), y]
    np.testing.assert_allclose(lp, ref, rtol=1e-14, atol=1e-14)
    u = np.full((3, 50), 0.7)
    np.testing.assert_allclose(grpo.token_logp(u, [0, 7, 49]), -np.log(50.0), rtol=1e-14)


def test_rho_one_closed_form():
    """old_logp = logp => rho = 1, nothing clipped: L = -(1/G) sum_i A_i, dlogits = A_i/(G R_i) (softmax - e_y)."""
    R, x, y, r = _case(2, G=5)
    G = 5
    lp = scipy.special.log_softmax(x, axis=1)[np.arange(x.shape[0]), y]
    A_raw = np.array([0.3, -1.1, 2.0, 0.25, -0.6])
    loss, dl, logp, clipped = grpo.grpo_token_loss(x, y, lp, R, r, G, 0.2, 0, G, A=A_raw)
    assert not clipped.any()
    assert abs(loss - (-A_raw.sum() / G)) < 1e-12
    soft = scipy.special.softmax(x, axis=1)
    resp = np.repeat(np.arange(G), R)
    onehot = np.zeros_like(x)
    onehot[np.arange(x.shape[0]), y] = 1
    want = (A_raw[resp] / (G * R[resp]))[:, None] * (soft - onehot)
    np.testing.assert_allclose(dl, want, rtol=1e-12, atol=1e-15)
    # normalised advantages sum to zero, so at rho = 1 the loss vanishes
    loss_n, *_ = grpo.grpo_token_loss(x, y, lp, R, r, G, 0.2, 0, G)
    assert abs(loss_n) < 1e-12


@pytest.mark.parametrize("A,delta,clipped_expected", [
    (1.5, +0.5, True),     # A > 0, rho > 1+eps  -> clipped, term (1+eps)A
    (1.5, -0.5, False),    # A > 0, rho < 1-eps  -> rho A, gradient flows
    (-1.5, -0.5, True),    # A < 0, rho < 1-eps  -> clipped, term (1-eps)A
    (-1.5, +0.5, False),   # A < 0, rho > 1+eps  -> rho A, gradient flows
    (1.5, 0.05, False),    # inside the band
])
def test_clip_branches(A, delta, clipped_expected):
    eps = 0.2
    g = np.random.default_rng(3)
    V, Rn = 9, 4
    x = g.standard_normal((Rn, V))
    y = g.integers(0, V, size=Rn)
    lp = scipy.special.log_softmax(x, axis=1)[np.arange(Rn), y]
    old = lp - delta                          # rho = exp(delta)
    rho = np.exp(delta)
    loss, dl, _, clipped = grpo.grpo_token_loss(x, y, old, [Rn], [0.0], 1, eps, 0, 1, A=[A])
    assert clipped.all() == clipped_expected and clipped.any() == clipped_expected
    if clipped_expected:
        term = (1 + eps) * A if A > 0 else (1 - eps) * A
        assert np.all(dl == 0.0)
    else:
        term = rho * A
        assert np.all(np.abs(dl).sum(1) > 0)
    assert abs(loss - (-term)) < 1e-12       # mean over R_i tokens of the same term, G = 1


def test_against_torch_autograd():
    import torch
    R, x, y, r = _case(4, G=4, V=13, sigma=1.0)
    g = np.random.default_rng(5)
    old = scipy.special.log_softmax(x, 1)[np.arange(x.shape[0]), y] + g.standard_normal(x.shape[0]) * 0.3
    eps, G = 0.2, 4
    loss, dl, logp, _ = grpo.grpo_token_loss(x, y, old, R, r, G, eps, 0, G)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    lpt = torch.log_softmax(xt, 1)[torch.arange(x.shape[0]), torch.tensor(y)]
    rho = torch.exp(lpt - torch.tensor(old))
    rr = torch.tensor(r)
    A = (rr - rr.mean()) / (rr.std(unbiased=False) + 1e-6)
    resp = torch.repeat_interleave(torch.arange(G), torch.tensor(R))
    At = A[resp]
    term = torch.minimum(rho * At, torch.clamp(rho, 1 - eps, 1 + eps) * At)
    L = -(term / (G * torch.tensor(R, dtype=torch.float64)[resp])).sum()
    L.backward()
    assert abs(loss - L.item()) < 1e-12
    np.testing.assert_allclose(dl, xt.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(logp, lpt.detach().numpy(), rtol=1e-14, atol=1e-14)


def test_finite_differences_v7():
    R, x, y, r = _case(6, G=3, V=7, sigma=1.0)
    g = np.random.default_rng(8)
    old = scipy.special.log_softmax(x, 1)[np.arange(x.shape[0]), y] + g.standard_normal(x.shape[0]) * 0.4
    G, eps = 3, 0.2
    _, dl, _, _ = grpo.grpo_token_loss(x, y, old, R, r, G, eps, 0, G)
    num = fd.grad(lambda z: grpo.grpo_token_loss(z, y, old, R, r, G, eps, 0, G)[0], x, h=1e-7)
    assert np.max(np.abs(num - dl)) < 1e-7 * max(1.0, np.max(np.abs(dl)))


def test_partial_range_sums_to_whole():
    R, x, y, r = _case(7, G=4)
    G = 4
    old = scipy.special.log_softmax(x, 1)[np.arange(x.shape[0]), y] + 0.1
    total, dl_all, *_ = grpo.grpo_token_loss(x, y, old, R, r, G, 0.2, 0, G)
    cu = np.concatenate([[0], np.cumsum(R)])
    acc = 0.0
    for i in range(G):
        li, dli, *_ = grpo.grpo_token_loss(x[cu[i]:cu[i + 1]], y[cu[i]:cu[i + 1]], old[cu[i]:cu[i + 1]], R, r, G,
                                           0.2, i, 1)
        acc += li
        np.testing.assert_array_equal(dli, dl_all[cu[i]:cu[i + 1]])
    assert abs(acc - total) < 1e-13


def test_advantage_properties():
    r = np.array([1.0, 0.0, 0.0, 1.0, 1.0, 0.0, 1.0, 1.0])
    A = grpo.advantages(r)
    assert abs(A.mean()) < 1e-15
    sd = np.sqrt(np.mean((r - r.mean()) ** 2))
    assert abs(np.mean(A ** 2) - (sd / (sd + 1e-6)) ** 2) < 1e-13
    assert abs(np.mean(A ** 2) - 1) < 1e-5
    # population std: G=2 with rewards {0,1} gives A = -1, +1 (up to the 1e-6 term)
    np.testing.assert_allclose(grpo.advantages([0.0, 1.0]), [-0.5 / 0.500001, 0.5 / 0.500001], rtol=1e-15)
    # all rewards equal => A == 0 exactly, loss 0, dlogits 0
    assert np.all(grpo.advantages([1.0, 1.0, 1.0]) == 0.0)
    # affine reward map r -> 2r - 1 (the pages' GLM run uses rewards in {-1, +1}) leaves A unchanged up to eps term
    np.testing.assert_allclose(grpo.advantages(2 * r - 1), A, rtol=2e-6)


def test_equal_rewards_zero_gradient():
    R, x, y, _ = _case(9, G=3)
    old = scipy.special.log_softmax(x, 1)[np.arange(x.shape[0]), y] + 0.7
    loss, dl, _, _ = grpo.grpo_token_loss(x, y, old, R, [1.0, 1.0, 1.0], 3, 0.2, 0, 3)
    assert loss == 0.0 and np.all(dl == 0.0)


def test_abs_term_scale_closed_forms():
    """S_abs = sum_i (1/(G R_i)) sum_t |term_it|, the scale of the loss bar, pinned by hand values.

    rho = 1: every term is A_i, so S_abs = (1/G) sum_i |A_i|; with G = 2 and rewards {0, 1} the
    population std is 1/2 and |A_i| = 0.5 / (0.5 + 1e-6). Clipped tokens: uniform logits over V = 4
    give logp = -log 4 exactly, and old = logp - log(rho) sets each token's ratio; with eps = 0.2 the
    terms are min(rho A, clip(rho) A). Unequal lengths catch a dropped 1/R_i, the clipped tokens a
    dropped clip, the negative advantage a dropped absolute value."""
    a = 0.5 / (0.5 + 1e-6)
    R = np.array([3, 5])
    rewards = np.array([0.0, 1.0])
    g = np.random.default_rng(7)
    x = g.standard_normal((8, 9))
    y = g.integers(0, 9, size=8)
    lp = grpo.token_logp(x, y)
    s = grpo.abs_term_scale(x, y, lp, R, rewards, 2, 0.2, 0, 2)
    assert abs(s - a) < 1e-12 * a
    # response 0 (reward 1, A = +a): rho = 1.5 (clipped: 1.2 a), 0.5 (0.5 a)
    # response 1 (reward 0, A = -a): rho = 0.5 (clipped: -0.8 a), 1.5 (-1.5 a), 1.0 (-a)
    R = np.array([2, 3])
    rewards = np.array([1.0, 0.0])
    rho = np.array([1.5, 0.5, 0.5, 1.5, 1.0])
    u = np.zeros((5, 4))
    y = np.array([0, 3, 1, 2, 0])
    old = -np.log(4.0) - np.log(rho)
    want_all = 0.5 * ((1.2 + 0.5) * a / 2 + (0.8 + 1.5 + 1.0) * a / 3)
    s = grpo.abs_term_scale(u, y, old, R, rewards, 2, 0.2, 0, 2)
    assert abs(s - want_all) < 1e-12 * want_all, (s, want_all)
    s1 = grpo.abs_term_scale(u[2:], y[2:], old[2:], R, rewards, 2, 0.2, 1, 1)
    want_1 = 0.5 * (0.8 + 1.5 + 1.0) * a / 3
    assert abs(s1 - want_1) < 1e-12 * want_1, (s1, want_1)
