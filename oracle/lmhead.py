"""LM head followed by the clipped-GRPO token objective, float64.  TEST INFRASTRUCTURE ONLY.

The token objective (LongStraw study notes, §1-1, the L_policy equation) is a function of each
token's logits row over the vocabulary. Those logits are the last hidden state times the
vocabulary projection: x_t = W h_t, i.e. logits = H W^T for hidden states H [T, d] and the
projection W [V, d]. This module composes that product with `grpo.grpo_token_loss`:

    logits = H W^T                         (rounded to bf16 when round_logits: the model's logits
                                            are bf16 tensors, formed from an fp32 accumulation)
    loss, dlogits, logp, clipped = grpo_token_loss(logits, ...)
    dH = dlogits W,   dW = dlogits^T H      (the chain rule through logits = H W^T)

The gradients are those of the loss as a function of the (rounded) logits; rounding is treated
as the identity in the backward pass, as a bf16 forward would be differentiated.
"""
from __future__ import annotations

import numpy as np

from oracle import grpo


def round_bf16(x):
    """x rounded to float32, then to bfloat16 (8 significant bits) to nearest, ties to even;
    returned as float64. Finite inputs only."""
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return bits.view(np.float32).astype(np.float64)


def lmhead_grpo_loss(H, W, targets, old_logp, R, rewards, G, eps, first, count, round_logits=True):
    """Share of L from responses [first, first+count) whose hidden rows are packed in H [T, d];
    W [V, d]. Returns (loss_share, dH [T, d], dW [V, d], logp [T], clipped [T] bool)."""
    H = np.asarray(H, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    logits = H @ W.T
    if round_logits:
        logits = round_bf16(logits)
    loss, dl, logp, clipped = grpo.grpo_token_loss(logits, targets, old_logp, R, rewards, G, eps, first, count)
    return loss, dl @ W, dl.T @ H, logp, clipped
