"""Clipped-GRPO token objective and its gradient w.r.t. logits, float64.  TEST INFRASTRUCTURE ONLY.

Policy objective (LongStraw study notes, §1-1, the L_policy equation):
    L = -(1/G) sum_i (1/R_i) sum_t min(rho_it A_i, clip(rho_it, 1-eps, 1+eps) A_i)
where rho_it is the ratio of current- to old-policy probability of the sampled token
(same section, the sentence after the equation), i.e. rho = exp(logp - old_logp).

logp is the log-softmax of the token's logits row at the sampled token (temperature 1,
full vocabulary). The group advantage is built from the group's rewards (§1-1 step 4,
§2-1 step 3); the pages give no formula, and the one used is
    A_i = (r_i - mean(r)) / (std(r) + 1e-6),  std = population standard deviation.

Gradient: min(rho A, clip(rho) A) follows rho A (gradient A * rho * dlogp) unless the
clipped branch is strictly smaller, which happens when A > 0 and rho > 1+eps or A < 0
and rho < 1-eps; then the term is constant and its gradient is zero. Equality counts
as the unclipped branch. d logp / d x = onehot(y) - softmax(x), so
    dL/dx_t = (A_i rho_t active_t / (G R_i)) * (softmax(x_t) - onehot(y_t)).
"""
from __future__ import annotations

import numpy as np


def advantages(rewards):
    r = np.asarray(rewards, dtype=np.float64)
    mean = r.sum() / r.size
    std = np.sqrt(np.sum((r - mean) ** 2) / r.size)
    return (r - mean) / (std + 1e-6)


def log_softmax_rows(x):
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=1, keepdims=True)
    return x - (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))


def token_logp(logits, targets):
    ls = log_softmax_rows(logits)
    return ls[np.arange(ls.shape[0]), np.asarray(targets)]


def grpo_token_loss(logits, targets, old_logp, R, rewards, G, eps, first, count, A=None):
    """Share of L from responses [first, first+count), their rows packed in `logits` [T, V].

    R, rewards: all G response lengths and rewards. A: optional override of the advantages
    (length G), used to test closed forms with un-normalised advantages.
    Returns (loss_share, dlogits [T,V], logp [T], clipped [T] bool).
    """
    R = np.asarray(R, dtype=np.int64)
    A = advantages(rewards) if A is None else np.asarray(A, dtype=np.float64)
    x = np.asarray(logits, dtype=np.float64)
    T, V = x.shape
    if T != int(R[first:first + count].sum()):
        raise ValueError("logits rows must equal the summed lengths of the selected responses")
    ls = log_softmax_rows(x)
    y = np.asarray(targets, dtype=np.int64)
    logp = ls[np.arange(T), y]
    resp = np.repeat(np.arange(first, first + count), R[first:first + count])
    A_t = A[resp]
    w_t = 1.0 / (G * R[resp].astype(np.float64))
    rho = np.exp(logp - np.asarray(old_logp, dtype=np.float64))
    unclipped = rho * A_t
    clipped_val = np.clip(rho, 1.0 - eps, 1.0 + eps) * A_t
    term = np.minimum(unclipped, clipped_val)
    is_clipped = clipped_val < unclipped
    loss = -np.sum(w_t * term)
    coef = np.where(is_clipped, 0.0, w_t * A_t * rho)
    soft = np.exp(ls)
    dlogits = coef[:, None] * soft
    dlogits[np.arange(T), y] -= coef
    return loss, dlogits, logp, is_clipped


def abs_term_scale(logits, targets, old_logp, R, rewards, G, eps, first, count):
    """S_abs = sum_i (1/(G R_i)) sum_t |term|: the scale against which the loss error is judged."""
    R = np.asarray(R, dtype=np.int64)
    A = advantages(rewards)
    logp = token_logp(logits, targets)
    resp = np.repeat(np.arange(first, first + count), R[first:first + count])
    rho = np.exp(logp - np.asarray(old_logp, dtype=np.float64))
    term = np.minimum(rho * A[resp], np.clip(rho, 1 - eps, 1 + eps) * A[resp])
    return float(np.sum(np.abs(term) / (G * R[resp])))
