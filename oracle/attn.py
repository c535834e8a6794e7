"""Replay attention by its plain definition, float64, CPU.  TEST INFRASTRUCTURE ONLY.

Setting (LongStraw study notes, §2-1 "serial policy replay" and §3-2 (2) "physical
page ownership"): a shared prompt of P tokens has per-layer keys/values K_P, V_P,
captured once without a graph. Each response i (R_i tokens) is replayed on its
own: its queries attend to every prompt key and, causally, to its own keys.

For response i, q head h, kv head k = h // (Hq/Hkv):
    Kbar = [K_P[:, k]; Ks_i[:, k]],  Vbar = [V_P[:, k]; Vs_i[:, k]]
    S[t, j] = scale * <Q_i[t, h], Kbar[j]>,  with suffix column P+s hidden when s > t
    LSE[t]  = log sum_visible exp(S[t, :])
    Pm      = exp(S - LSE)            (exact softmax, not an online update)
    O[t, h] = Pm[t, :] @ Vbar
Backward, given dO (the standard softmax-attention derivative):
    dPm = dO_h Vbar^T,  Dlt[t] = <dO_h[t], O_h[t]>,  dS = Pm * (dPm - Dlt)
    dQ_h = scale * dS Kbar,  dKbar += scale * dS^T Q_h,  dVbar += Pm^T dO_h
The prompt rows of dKbar/dVbar are the prompt-side gradient (the d l / d z_P term
of the gradient decomposition in §2-2); they are summed over heads and over the
responses of the group, as serial replay accumulates them before the single
finalisation (§2-1 step 5). The suffix rows are the response's own dKs/dVs.

Query rows are processed a chunk at a time; each row's softmax is complete within
its chunk, so chunking changes nothing but memory use.
"""
from __future__ import annotations

import numpy as np


def _chunk_rows(ncols: int) -> int:
    return int(max(1, min(256, (1 << 24) // max(1, ncols))))


def _head_operands(Kp, Vp, Ks, Vs, r0, r1, k):
    Kbar = np.concatenate([Kp[:, k, :], Ks[r0:r1, k, :]], axis=0)
    Vbar = np.concatenate([Vp[:, k, :], Vs[r0:r1, k, :]], axis=0)
    return Kbar, Vbar


def _scores(q_rows, Kbar, P, t_rel, scale):
    """S for query rows whose in-response positions are t_rel; hidden entries are -inf."""
    S = scale * (q_rows @ Kbar.T)
    R = Kbar.shape[0] - P
    s_idx = np.arange(R)
    hidden = s_idx[None, :] > t_rel[:, None]
    S[:, P:][hidden] = -np.inf
    return S


def _softmax_rows(S):
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]
    return e / z, lse


def replay_attn_fwd(Kp, Vp, Q, Ks, Vs, cu_seqlens, scale, rows=None):
    """Forward replay attention.

    Kp [P,Hkv,Dqk], Vp [P,Hkv,Dv], Q [T,Hq,Dqk], Ks [T,Hkv,Dqk], Vs [T,Hkv,Dv] (float64),
    cu_seqlens [n_resp+1] (response i owns packed rows cu[i]:cu[i+1]).
    rows: optional sorted array of packed row indices; only those rows are computed.
    Returns O [T,Hq,Dv] and LSE [Hq,T] (rows not computed are NaN).
    """
    P, Hkv, _ = Kp.shape
    T, Hq, _ = Q.shape
    Dv = Vp.shape[2]
    g = Hq // Hkv
    O = np.full((T, Hq, Dv), np.nan)
    LSE = np.full((Hq, T), np.nan)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(len(cu) - 1):
        r0, r1 = int(cu[i]), int(cu[i + 1])
        tsel = np.arange(r0, r1) if rows is None else np.asarray([t for t in rows if r0 <= t < r1], dtype=np.int64)
        if tsel.size == 0:
            continue
        for h in range(Hq):
            k = h // g
            Kbar, Vbar = _head_operands(Kp, Vp, Ks, Vs, r0, r1, k)
            step = _chunk_rows(Kbar.shape[0])
            for c in range(0, tsel.size, step):
                t = tsel[c:c + step]
                S = _scores(Q[t, h, :], Kbar, P, t - r0, scale)
                Pm, lse = _softmax_rows(S)
                O[t, h, :] = Pm @ Vbar
                LSE[h, t] = lse
    return O, LSE


def replay_attn_bwd(Kp, Vp, Q, Ks, Vs, dO, cu_seqlens, scale, dKp_acc=None, dVp_acc=None):
    """Backward replay attention.

    Returns dQ [T,Hq,Dqk], dKs [T,Hkv,Dqk], dVs [T,Hkv,Dv]. If dKp_acc/dVp_acc ([P,Hkv,Dqk] /
    [P,Hkv,Dv] float64) are given, the prompt-side gradient of every response is ADDED to them in
    place (exact prompt-gradient mode); if both are None the prompt side is not formed
    (response-only closure, the stop-gradient prompt boundary of §2-2).
    """
    if (dKp_acc is None) != (dVp_acc is None):
        raise ValueError("dKp_acc and dVp_acc must both be given or both be None")
    P, Hkv, Dqk = Kp.shape
    T, Hq, _ = Q.shape
    g = Hq // Hkv
    dQ = np.zeros_like(Q, dtype=np.float64)
    dKs = np.zeros((T, Hkv, Dqk))
    dVs = np.zeros((T, Hkv, Vp.shape[2]))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for i in range(len(cu) - 1):
        r0, r1 = int(cu[i]), int(cu[i + 1])
        if r1 <= r0:
            continue
        for h in range(Hq):
            k = h // g
            Kbar, Vbar = _head_operands(Kp, Vp, Ks, Vs, r0, r1, k)
            dKbar = np.zeros_like(Kbar)
            dVbar = np.zeros_like(Vbar)
            step = _chunk_rows(Kbar.shape[0])
            for c0 in range(r0, r1, step):
                t = np.arange(c0, min(r1, c0 + step))
                q = Q[t, h, :]
                do = dO[t, h, :]
                S = _scores(q, Kbar, P, t - r0, scale)
                Pm, _ = _softmax_rows(S)
                o = Pm @ Vbar
                dPm = do @ Vbar.T
                dlt = np.sum(do * o, axis=1)
                dS = Pm * (dPm - dlt[:, None])
                dQ[t, h, :] = scale * (dS @ Kbar)
                dKbar += scale * (dS.T @ q)
                dVbar += Pm.T @ do
            dKs[r0:r1, k, :] += dKbar[P:]
            dVs[r0:r1, k, :] += dVbar[P:]
            if dKp_acc is not None:
                dKp_acc[:, k, :] += dKbar[:P]
                dVp_acc[:, k, :] += dVbar[:P]
    return dQ, dKs, dVs


def replay_attn_bwd_rows(Kp, Vp, Q, Ks, Vs, dO, cu_seqlens, scale, rows):
    """dQ for selected packed rows only (each row's dQ depends on that row alone). Returns [len(rows),Hq,Dqk]."""
    P, Hkv, _ = Kp.shape
    T, Hq, Dqk = Q.shape
    g = Hq // Hkv
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, Hq, Dqk))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for n, t in enumerate(rows):
        i = int(np.searchsorted(cu, t, side="right") - 1)
        r0, r1 = int(cu[i]), int(cu[i + 1])
        for h in range(Hq):
            k = h // g
            Kbar, Vbar = _head_operands(Kp, Vp, Ks, Vs, r0, r1, k)
            S = _scores(Q[[t], h, :], Kbar, P, np.asarray([t - r0]), scale)
            Pm, _ = _softmax_rows(S)
            o = Pm @ Vbar
            do = dO[[t], h, :]
            dS = Pm * (do @ Vbar.T - np.sum(do * o, axis=1)[:, None])
            out[n, h, :] = scale * (dS @ Kbar)[0]
    return out
