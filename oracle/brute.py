"""Independent attention formulations used to pin `oracle.attn`.  TEST INFRASTRUCTURE ONLY.

Replay (LongStraw study notes, §2-1 step 4 and §2-2) claims to compute, for each
response, exactly what ordinary causal attention over the concatenated sequence
[prompt; response] computes for the response's rows. These routines write that
ordinary attention down directly, in two ways that share nothing with `attn`:

* `causal_concat_*`: textbook causal attention over the whole concatenated
  sequence (dense L x L scores, lower-triangular mask), numpy float64; the prompt
  rows get zero queries and their outputs are discarded.
* `torch_concat_*` / `torch_tree_batch_grads`: the same through the library routine
  torch.nn.functional.scaled_dot_product_attention in float64 on the CPU, with
  torch autograd for the backward. The tree-masked batch puts the whole group
  [prompt; Y_1; ...; Y_G] in one sequence where Y_i sees the prompt and, causally,
  itself: the conventional whole-group backward that serial replay replaces (§1-2 (3)).
"""
from __future__ import annotations

import numpy as np


def causal_concat_fwd(Kp, Vp, q_resp, Ks, Vs, scale):
    """One response. Kp [P,Hkv,D], q_resp [R,Hq,D], Ks [R,Hkv,D] ... Returns O [R,Hq,Dv], LSE [Hq,R]."""
    P, Hkv, Dqk = Kp.shape
    R, Hq, _ = q_resp.shape
    g = Hq // Hkv
    L = P + R
    K = np.concatenate([Kp, Ks], axis=0)
    V = np.concatenate([Vp, Vs], axis=0)
    Qf = np.concatenate([np.zeros((P, Hq, Dqk)), q_resp], axis=0)
    O = np.zeros((R, Hq, V.shape[2]))
    LSE = np.zeros((Hq, R))
    for h in range(Hq):
        k = h // g
        S = scale * (Qf[:, h, :] @ K[:, k, :].T)
        S[np.triu(np.ones((L, L), dtype=bool), 1)] = -np.inf
        for i in range(P, L):
            row = S[i]
            m = np.max(row)
            w = np.exp(row - m)
            z = np.sum(w)
            O[i - P, h] = (w / z) @ V[:, k, :]
            LSE[h, i - P] = m + np.log(z)
    return O, LSE


def _torch():
    import torch
    return torch


def torch_concat_fwd_bwd(Kp, Vp, q_resp, Ks, Vs, dO_resp, scale):
    """Forward + backward through float64 SDPA on [prompt; response] with is_causal=True.

    Returns O [R,Hq,Dv], dQ [R,Hq,D], dKp [P,Hkv,D], dVp [P,Hkv,Dv], dKs [R,Hkv,D], dVs [R,Hkv,Dv].
    """
    torch = _torch()
    P, Hkv, Dqk = Kp.shape
    R, Hq, _ = q_resp.shape
    g = Hq // Hkv
    K = torch.tensor(np.concatenate([Kp, Ks], 0), dtype=torch.float64, requires_grad=True)
    V = torch.tensor(np.concatenate([Vp, Vs], 0), dtype=torch.float64, requires_grad=True)
    qr = torch.tensor(q_resp, dtype=torch.float64, requires_grad=True)
    Qf = torch.cat([torch.zeros(P, Hq, Dqk, dtype=torch.float64), qr], 0)
    heads = torch.arange(Hq) // g
    Kh = K[:, heads, :].permute(1, 0, 2)
    Vh = V[:, heads, :].permute(1, 0, 2)
    Qh = Qf.permute(1, 0, 2)
    Oh = torch.nn.functional.scaled_dot_product_attention(Qh, Kh, Vh, is_causal=True, scale=scale)
    O = Oh.permute(1, 0, 2)[P:]
    O.backward(torch.tensor(dO_resp, dtype=torch.float64))
    return (O.detach().numpy(), qr.grad.numpy(), K.grad[:P].numpy(), V.grad[:P].numpy(),
            K.grad[P:].numpy(), V.grad[P:].numpy())


def torch_tree_batch_grads(Kp, Vp, Q, Ks, Vs, dO, cu_seqlens, scale):
    """Whole group in one tree-masked sequence [prompt; Y_1; ...; Y_n]; float64 SDPA + autograd.

    Returns O [T,Hq,Dv], dQ [T,Hq,D], dKp [P,Hkv,D], dVp [P,Hkv,Dv], dKs [T,Hkv,D], dVs [T,Hkv,Dv].
    """
    torch = _torch()
    P, Hkv, Dqk = Kp.shape
    T, Hq, _ = Q.shape
    g = Hq // Hkv
    L = P + T
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seg = np.full(L, -1)
    pos = np.zeros(L, dtype=np.int64)
    pos[:P] = np.arange(P)
    for i in range(len(cu) - 1):
        seg[P + cu[i]:P + cu[i + 1]] = i
        pos[P + cu[i]:P + cu[i + 1]] = np.arange(cu[i + 1] - cu[i])
    allow = np.zeros((L, L), dtype=bool)
    for a in range(L):
        for b in range(L):
            if seg[b] == -1:
                allow[a, b] = seg[a] != -1 or b <= a      # prompt keys: all for responses, causal for prompt
            else:
                allow[a, b] = seg[a] == seg[b] and pos[b] <= pos[a]
    K = torch.tensor(np.concatenate([Kp, Ks], 0), dtype=torch.float64, requires_grad=True)
    V = torch.tensor(np.concatenate([Vp, Vs], 0), dtype=torch.float64, requires_grad=True)
    qr = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    Qf = torch.cat([torch.zeros(P, Hq, Dqk, dtype=torch.float64), qr], 0)
    heads = torch.arange(Hq) // g
    Oh = torch.nn.functional.scaled_dot_product_attention(
        Qf.permute(1, 0, 2), K[:, heads, :].permute(1, 0, 2), V[:, heads, :].permute(1, 0, 2),
        attn_mask=torch.tensor(allow), scale=scale)
    O = Oh.permute(1, 0, 2)[P:]
    O.backward(torch.tensor(dO, dtype=torch.float64))
    return (O.detach().numpy(), qr.grad.numpy(), K.grad[:P].numpy(), V.grad[:P].numpy(),
            K.grad[P:].numpy(), V.grad[P:].numpy())
