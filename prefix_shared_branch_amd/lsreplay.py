"""Python binding of liblsreplay (ctypes). Argument marshalling only: every step of the
computation runs in the library's HIP kernels. PyTorch supplies device memory and the
current stream; nothing else of torch is used.

The functions carry the C entry points' names (include/ls_replay.h) and take torch tensors.
If the library is not built the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsreplay.so")

LS_OK, LS_ERR_INVALID_ARG, LS_ERR_UNSUPPORTED, LS_ERR_WORKSPACE, LS_ERR_HIP = 0, -1, -2, -3, -4
LS_MAX_RESPONSES_PER_CALL = 64
LS_NOALLOC_MAX_ROWS = 1048576
EXPORTED = ("ls_replay_attn_workspace_bytes", "ls_replay_attn_fwd", "ls_replay_attn_bwd",
            "ls_replay_attn_block_workspace_bytes", "ls_replay_attn_fwd_block", "ls_replay_attn_bwd_block",
            "ls_grpo_workspace_bytes", "ls_grpo_token_loss", "ls_grpo_token_loss_noalloc",
            "ls_grpo_lmhead_workspace_bytes",
            "ls_grpo_lmhead_loss", "ls_status_string", "ls_kernel_timer_start", "ls_kernel_timer_stop")
LS_KERNEL_ATTN_FWD, LS_KERNEL_DKDV_PROMPT, LS_KERNEL_DQ, LS_KERNEL_GRPO_ROWS = 0, 1, 2, 3


class LsError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {ls_status_string(code)} ({code})")
        self.code = code


class AttnDesc(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("ldk", ctypes.c_int64),
                ("ldv", ctypes.c_int64), ("softmax_scale", ctypes.c_float)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with prefix_shared_branch_amd/build.py "
                              "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        pdesc = ctypes.POINTER(AttnDesc)
        pi32 = ctypes.POINTER(ctypes.c_int32)
        pf32 = ctypes.POINTER(ctypes.c_float)
        L.ls_status_string.restype = ctypes.c_char_p
        L.ls_status_string.argtypes = [ctypes.c_int]
        L.ls_replay_attn_workspace_bytes.restype = ctypes.c_int
        L.ls_replay_attn_workspace_bytes.argtypes = [pdesc, i32, pi32, i32, ctypes.POINTER(sz)]
        L.ls_replay_attn_fwd.restype = ctypes.c_int
        L.ls_replay_attn_fwd.argtypes = [vp, pdesc, vp, vp, i32, pi32, vp, vp, vp, vp, vp, vp, vp, sz]
        L.ls_replay_attn_bwd.restype = ctypes.c_int
        L.ls_replay_attn_bwd.argtypes = [vp, pdesc, vp, vp, i32, pi32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz]
        L.ls_replay_attn_block_workspace_bytes.restype = ctypes.c_int
        L.ls_replay_attn_block_workspace_bytes.argtypes = [pdesc, i32, i32, i32, ctypes.POINTER(sz)]
        L.ls_replay_attn_fwd_block.restype = ctypes.c_int
        L.ls_replay_attn_fwd_block.argtypes = [vp, pdesc, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz]
        L.ls_replay_attn_bwd_block.restype = ctypes.c_int
        L.ls_replay_attn_bwd_block.argtypes = [vp, pdesc, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, vp, vp, sz]
        L.ls_grpo_workspace_bytes.restype = ctypes.c_int
        L.ls_grpo_workspace_bytes.argtypes = [i64, i32, ctypes.POINTER(sz)]
        L.ls_grpo_token_loss.restype = ctypes.c_int
        L.ls_grpo_token_loss.argtypes = [vp, i32, i32, pi32, pf32, f32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz]
        L.ls_grpo_token_loss_noalloc.restype = ctypes.c_int
        L.ls_grpo_token_loss_noalloc.argtypes = [vp, i32, i32, pi32, pf32, f32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.ls_grpo_lmhead_workspace_bytes.restype = ctypes.c_int
        L.ls_grpo_lmhead_workspace_bytes.argtypes = [i64, i32, i32, ctypes.POINTER(sz)]
        L.ls_grpo_lmhead_loss.restype = ctypes.c_int
        L.ls_grpo_lmhead_loss.argtypes = [vp, i32, i32, i32, pi32, pf32, f32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, sz]
        L.ls_kernel_timer_start.restype = ctypes.c_int
        L.ls_kernel_timer_start.argtypes = [i32]
        L.ls_kernel_timer_stop.restype = ctypes.c_int
        L.ls_kernel_timer_stop.argtypes = [pf32, pi32]
        _lib = L
    return _lib


def ls_status_string(code: int) -> str:
    return lib().ls_status_string(int(code)).decode()


def _check(fn, code):
    if code != LS_OK:
        raise LsError(fn, code)


def _i32_array(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _f32_array(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _kv_stride(t, name, d):
    if t.dim() != 3 or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != d):
        raise ValueError(f"{name} must be [tokens, heads, {d}] with unit last stride and head stride {d}")
    return t.stride(0)


def make_desc(q, kp, vp, ks, vs, scale=None) -> AttnDesc:
    """Descriptor from tensor shapes/strides: q [T,Hq,Dqk], kp/ks [*,Hkv,Dqk], vp/vs [*,Hkv,Dv] (row strides ldk/ldv)."""
    T, Hq, Dqk = q.shape
    Hkv, Dv = kp.shape[1], vp.shape[2]
    ldk = _kv_stride(ks, "ks", Dqk)
    ldv = _kv_stride(vs, "vs", Dv)
    if kp.shape[0] > 0 and (_kv_stride(kp, "kp", Dqk) != ldk or _kv_stride(vp, "vp", Dv) != ldv):
        raise ValueError("prompt and suffix K/V must share the row strides ldk/ldv")
    d = AttnDesc()
    d.P, d.Hq, d.Hkv, d.Dqk, d.Dv = kp.shape[0], Hq, Hkv, Dqk, Dv
    d.ldk, d.ldv = ldk, ldv
    d.softmax_scale = float(1.0 / np.sqrt(Dqk)) if scale is None else float(scale)
    return d


def ls_replay_attn_workspace_bytes(desc: AttnDesc, cu_seqlens, which: int) -> int:
    cu, cup = _i32_array(cu_seqlens)
    out = ctypes.c_size_t(0)
    _check("ls_replay_attn_workspace_bytes",
           lib().ls_replay_attn_workspace_bytes(ctypes.byref(desc), len(cu) - 1, cup, int(which), ctypes.byref(out)))
    return int(out.value)


def _workspace(nbytes, device, workspace):
    import torch
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _check_tensor(t, name, dtype, shape=None):
    if t.dtype != dtype or not t.is_cuda:
        raise ValueError(f"{name} must be a {dtype} CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_o_lo(o_lo, shape):
    import torch
    if o_lo is not None:
        _check_tensor(o_lo, "o_lo", torch.bfloat16, shape)
        if not o_lo.is_contiguous():
            raise ValueError("o_lo must be contiguous")


def ls_replay_attn_fwd(q, ks, vs, kp, vp, cu_seqlens, scale=None, out=None, lse=None, workspace=None, o_lo=None):
    """Replay attention forward. Returns (O [T,Hq,Dv] bf16, LSE [Hq,T] fp32); fills o_lo (bf16
    [T,Hq,Dv], the rounding residual of O for the backward's Delta) when it is given."""
    import torch
    desc = make_desc(q, kp, vp, ks, vs, scale)
    T, Hq = q.shape[0], q.shape[1]
    for n, t in (("q", q), ("ks", ks), ("vs", vs), ("kp", kp), ("vp", vp)):
        _check_tensor(t, n, torch.bfloat16)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    out = torch.empty(T, Hq, desc.Dv, dtype=torch.bfloat16, device=q.device) if out is None else out
    lse = torch.empty(Hq, T, dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(out, "out", torch.bfloat16, (T, Hq, desc.Dv))
    _check_tensor(lse, "lse", torch.float32, (Hq, T))
    _check_o_lo(o_lo, (T, Hq, desc.Dv))
    cu, cup = _i32_array(cu_seqlens)
    nbytes = ls_replay_attn_workspace_bytes(desc, cu, 0)
    ws = _workspace(nbytes, q.device, workspace)
    _check("ls_replay_attn_fwd", lib().ls_replay_attn_fwd(
        _stream(), ctypes.byref(desc), _ptr(kp) if kp.numel() else None, _ptr(vp) if vp.numel() else None,
        len(cu) - 1, cup, _ptr(q), _ptr(ks), _ptr(vs), _ptr(out), _ptr(lse), _ptr(o_lo), _ptr(ws), ws.numel()))
    return out, lse


def ls_replay_attn_bwd(q, ks, vs, kp, vp, cu_seqlens, o, lse, do, dkp_accum=None, dvp_accum=None, scale=None,
                       dq=None, dks=None, dvs=None, workspace=None, o_lo=None):
    """Replay attention backward. Adds into dkp_accum/dvp_accum (fp32) when given (exact
    prompt-gradient mode); both None = response-only closure. o_lo: the forward's residual of O,
    or None. Returns (dQ, dKs, dVs) bf16."""
    import torch
    desc = make_desc(q, kp, vp, ks, vs, scale)
    T, Hq = q.shape[0], q.shape[1]
    for n, t in (("q", q), ("ks", ks), ("vs", vs), ("kp", kp), ("vp", vp), ("o", o), ("do", do)):
        _check_tensor(t, n, torch.bfloat16)
    _check_tensor(lse, "lse", torch.float32, (Hq, T))
    if (dkp_accum is None) != (dvp_accum is None):
        raise ValueError("dkp_accum and dvp_accum must both be given or both be None")
    if dkp_accum is not None:
        _check_tensor(dkp_accum, "dkp_accum", torch.float32, (desc.P, desc.Hkv, desc.Dqk))
        _check_tensor(dvp_accum, "dvp_accum", torch.float32, (desc.P, desc.Hkv, desc.Dv))
        if not (dkp_accum.is_contiguous() and dvp_accum.is_contiguous()):
            raise ValueError("accumulators must be contiguous")
    for n, t in (("q", q), ("o", o), ("do", do)):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    dq = torch.empty(T, Hq, desc.Dqk, dtype=torch.bfloat16, device=q.device) if dq is None else dq
    dks = torch.empty(T, desc.Hkv, desc.Dqk, dtype=torch.bfloat16, device=q.device) if dks is None else dks
    dvs = torch.empty(T, desc.Hkv, desc.Dv, dtype=torch.bfloat16, device=q.device) if dvs is None else dvs
    cu, cup = _i32_array(cu_seqlens)
    _check_o_lo(o_lo, (T, Hq, desc.Dv))
    nbytes = ls_replay_attn_workspace_bytes(desc, cu, 1 if dkp_accum is not None else 2)
    ws = _workspace(nbytes, q.device, workspace)
    _check("ls_replay_attn_bwd", lib().ls_replay_attn_bwd(
        _stream(), ctypes.byref(desc), _ptr(kp) if kp.numel() else None, _ptr(vp) if vp.numel() else None,
        len(cu) - 1, cup, _ptr(q), _ptr(ks), _ptr(vs), _ptr(o), _ptr(lse), _ptr(o_lo), _ptr(do), _ptr(dq), _ptr(dks),
        _ptr(dvs), _ptr(dkp_accum), _ptr(dvp_accum), _ptr(ws), ws.numel()))
    return dq, dks, dvs


def ls_replay_attn_block_workspace_bytes(desc: AttnDesc, q0: int, nq: int, which: int) -> int:
    out = ctypes.c_size_t(0)
    _check("ls_replay_attn_block_workspace_bytes",
           lib().ls_replay_attn_block_workspace_bytes(ctypes.byref(desc), int(q0), int(nq), int(which),
                                                      ctypes.byref(out)))
    return int(out.value)


def ls_replay_attn_fwd_block(q, ks, vs, kp, vp, q0, scale=None, out=None, lse=None, workspace=None, o_lo=None):
    """Forward of rows q0 .. q0+nq-1 of one response (q [nq,Hq,Dqk]; ks/vs hold the response's keys
    0 .. q0+nq-1). Returns (O [nq,Hq,Dv] bf16, LSE [Hq,nq] fp32)."""
    import torch
    desc = make_desc(q, kp, vp, ks, vs, scale)
    nq, Hq = q.shape[0], q.shape[1]
    for n, t in (("q", q), ("ks", ks), ("vs", vs), ("kp", kp), ("vp", vp)):
        _check_tensor(t, n, torch.bfloat16)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if ks.shape[0] != q0 + nq or vs.shape[0] != q0 + nq:
        raise ValueError(f"ks/vs must hold the response's keys 0 .. q0+nq-1 ({q0 + nq} rows)")
    out = torch.empty(nq, Hq, desc.Dv, dtype=torch.bfloat16, device=q.device) if out is None else out
    lse = torch.empty(Hq, nq, dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(out, "out", torch.bfloat16, (nq, Hq, desc.Dv))
    _check_tensor(lse, "lse", torch.float32, (Hq, nq))
    _check_o_lo(o_lo, (nq, Hq, desc.Dv))
    ws = _workspace(ls_replay_attn_block_workspace_bytes(desc, q0, nq, 0), q.device, workspace)
    _check("ls_replay_attn_fwd_block", lib().ls_replay_attn_fwd_block(
        _stream(), ctypes.byref(desc), _ptr(kp) if kp.numel() else None, _ptr(vp) if vp.numel() else None,
        int(q0), int(nq), _ptr(q), _ptr(ks), _ptr(vs), _ptr(out), _ptr(lse), _ptr(o_lo), _ptr(ws), ws.numel()))
    return out, lse


def ls_replay_attn_bwd_block(q, ks, vs, kp, vp, q0, o, lse, do, dks_accum, dvs_accum, dkp_accum=None,
                             dvp_accum=None, scale=None, dq=None, workspace=None, o_lo=None):
    """Backward of one block: returns dQ [nq,Hq,Dqk] bf16 and ADDS the block's key gradients into
    dks_accum/dvs_accum (fp32 [q0+nq,Hkv,*]) and, in exact mode, into dkp_accum/dvp_accum."""
    import torch
    desc = make_desc(q, kp, vp, ks, vs, scale)
    nq, Hq = q.shape[0], q.shape[1]
    for n, t in (("q", q), ("ks", ks), ("vs", vs), ("kp", kp), ("vp", vp), ("o", o), ("do", do)):
        _check_tensor(t, n, torch.bfloat16)
    _check_tensor(lse, "lse", torch.float32, (Hq, nq))
    if ks.shape[0] != q0 + nq or vs.shape[0] != q0 + nq:
        raise ValueError(f"ks/vs must hold the response's keys 0 .. q0+nq-1 ({q0 + nq} rows)")
    _check_tensor(dks_accum, "dks_accum", torch.float32, (q0 + nq, desc.Hkv, desc.Dqk))
    _check_tensor(dvs_accum, "dvs_accum", torch.float32, (q0 + nq, desc.Hkv, desc.Dv))
    if (dkp_accum is None) != (dvp_accum is None):
        raise ValueError("dkp_accum and dvp_accum must both be given or both be None")
    if dkp_accum is not None:
        _check_tensor(dkp_accum, "dkp_accum", torch.float32, (desc.P, desc.Hkv, desc.Dqk))
        _check_tensor(dvp_accum, "dvp_accum", torch.float32, (desc.P, desc.Hkv, desc.Dv))
    for n, t in (("q", q), ("o", o), ("do", do), ("dks_accum", dks_accum), ("dvs_accum", dvs_accum)):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    _check_o_lo(o_lo, (nq, Hq, desc.Dv))
    dq = torch.empty(nq, Hq, desc.Dqk, dtype=torch.bfloat16, device=q.device) if dq is None else dq
    ws = _workspace(ls_replay_attn_block_workspace_bytes(desc, q0, nq, 1 if dkp_accum is not None else 2),
                    q.device, workspace)
    _check("ls_replay_attn_bwd_block", lib().ls_replay_attn_bwd_block(
        _stream(), ctypes.byref(desc), _ptr(kp) if kp.numel() else None, _ptr(vp) if vp.numel() else None,
        int(q0), int(nq), _ptr(q), _ptr(ks), _ptr(vs), _ptr(o), _ptr(lse), _ptr(o_lo), _ptr(do), _ptr(dq),
        _ptr(dks_accum), _ptr(dvs_accum), _ptr(dkp_accum), _ptr(dvp_accum), _ptr(ws), ws.numel()))
    return dq


def ls_grpo_workspace_bytes(T: int, V: int) -> int:
    out = ctypes.c_size_t(0)
    _check("ls_grpo_workspace_bytes", lib().ls_grpo_workspace_bytes(int(T), int(V), ctypes.byref(out)))
    return int(out.value)


def ls_grpo_token_loss(logits, targets, old_logp, R, rewards, eps, first, count, loss_accum, dlogits=None,
                       logp_out=None, clipped_out=None, workspace=None, scoring_only=False):
    """Clipped-GRPO loss share of responses [first, first+count) added into loss_accum (fp32 [1]);
    returns dlogits (bf16 [T,V]), or None with scoring_only (no gradient: log-probs, clip flags and
    the loss share only)."""
    import torch
    T, V = logits.shape
    _check_tensor(logits, "logits", torch.bfloat16)
    _check_tensor(targets, "targets", torch.int32, (T,))
    _check_tensor(old_logp, "old_logp", torch.float32, (T,))
    _check_tensor(loss_accum, "loss_accum", torch.float32)
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    if scoring_only:
        if dlogits is not None:
            raise ValueError("scoring_only takes no dlogits buffer")
    else:
        dlogits = torch.empty_like(logits) if dlogits is None else dlogits
        _check_tensor(dlogits, "dlogits", torch.bfloat16, (T, V))
    if logp_out is not None:
        _check_tensor(logp_out, "logp_out", torch.float32, (T,))
    if clipped_out is not None:
        _check_tensor(clipped_out, "clipped_out", torch.uint8, (T,))
    Ra, Rp = _i32_array(R)
    ra, rp = _f32_array(rewards)
    ws = _workspace(ls_grpo_workspace_bytes(T, V), logits.device, workspace)
    _check("ls_grpo_token_loss", lib().ls_grpo_token_loss(
        _stream(), V, len(Ra), Rp, rp, float(eps), int(first), int(count), _ptr(logits), _ptr(targets),
        _ptr(old_logp), _ptr(dlogits), _ptr(loss_accum), _ptr(logp_out), _ptr(clipped_out), _ptr(ws), ws.numel()))
    return dlogits


def ls_grpo_token_loss_noalloc(logits, targets, old_logp, R, rewards, eps, first, count, loss_accum, dlogits,
                               logp_out=None, clipped_out=None):
    """ls_grpo_token_loss with the library's fixed per-GPU scratch array instead of a workspace: the
    caller passes every output (dlogits, or None for scoring only); nothing is allocated."""
    import torch
    T, V = logits.shape
    _check_tensor(logits, "logits", torch.bfloat16)
    _check_tensor(targets, "targets", torch.int32, (T,))
    _check_tensor(old_logp, "old_logp", torch.float32, (T,))
    _check_tensor(loss_accum, "loss_accum", torch.float32)
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    if dlogits is not None:
        _check_tensor(dlogits, "dlogits", torch.bfloat16, (T, V))
    if logp_out is not None:
        _check_tensor(logp_out, "logp_out", torch.float32, (T,))
    if clipped_out is not None:
        _check_tensor(clipped_out, "clipped_out", torch.uint8, (T,))
    Ra, Rp = _i32_array(R)
    ra, rp = _f32_array(rewards)
    _check("ls_grpo_token_loss_noalloc", lib().ls_grpo_token_loss_noalloc(
        _stream(), V, len(Ra), Rp, rp, float(eps), int(first), int(count), _ptr(logits), _ptr(targets),
        _ptr(old_logp), _ptr(dlogits), _ptr(loss_accum), _ptr(logp_out), _ptr(clipped_out)))
    return dlogits


def ls_grpo_lmhead_workspace_bytes(T: int, V: int, d: int) -> int:
    out = ctypes.c_size_t(0)
    _check("ls_grpo_lmhead_workspace_bytes", lib().ls_grpo_lmhead_workspace_bytes(int(T), int(V), int(d),
                                                                                  ctypes.byref(out)))
    return int(out.value)


def ls_grpo_lmhead_loss(H, W, targets, old_logp, R, rewards, eps, first, count, loss_accum, dW_accum=None,
                        dH=None, logp_out=None, clipped_out=None, workspace=None, scoring_only=False):
    """LM head (logits = H W^T, chunked) fused with the clipped-GRPO loss of responses [first, first+count):
    adds the loss share into loss_accum and dL/dW into dW_accum (fp32 [V, d]); returns dH (bf16 [T, d]),
    or None with scoring_only."""
    import torch
    T, d = H.shape
    V = W.shape[0]
    _check_tensor(H, "H", torch.bfloat16)
    _check_tensor(W, "W", torch.bfloat16, (V, d))
    _check_tensor(targets, "targets", torch.int32, (T,))
    _check_tensor(old_logp, "old_logp", torch.float32, (T,))
    _check_tensor(loss_accum, "loss_accum", torch.float32)
    if not (H.is_contiguous() and W.is_contiguous()):
        raise ValueError("H and W must be contiguous")
    if scoring_only:
        if dH is not None or dW_accum is not None:
            raise ValueError("scoring_only takes no gradient buffers")
    else:
        if dW_accum is None:
            raise ValueError("dW_accum (fp32 [V, d], zeroed by the caller) is required")
        _check_tensor(dW_accum, "dW_accum", torch.float32, (V, d))
        dH = torch.empty_like(H) if dH is None else dH
        _check_tensor(dH, "dH", torch.bfloat16, (T, d))
    if logp_out is not None:
        _check_tensor(logp_out, "logp_out", torch.float32, (T,))
    if clipped_out is not None:
        _check_tensor(clipped_out, "clipped_out", torch.uint8, (T,))
    Ra, Rp = _i32_array(R)
    ra, rp = _f32_array(rewards)
    ws = _workspace(ls_grpo_lmhead_workspace_bytes(T, V, d), H.device, workspace)
    _check("ls_grpo_lmhead_loss", lib().ls_grpo_lmhead_loss(
        _stream(), V, d, len(Ra), Rp, rp, float(eps), int(first), int(count), _ptr(H), _ptr(W), _ptr(targets),
        _ptr(old_logp), _ptr(loss_accum), _ptr(dH), _ptr(dW_accum), _ptr(logp_out), _ptr(clipped_out), _ptr(ws),
        ws.numel()))
    return dH


def ls_kernel_timer_start(kernel: int) -> None:
    """Arm the library's kernel timer for one kernel (an LS_KERNEL_* id)."""
    _check("ls_kernel_timer_start", lib().ls_kernel_timer_start(int(kernel)))


def ls_kernel_timer_stop():
    """Disarm the kernel timer; returns (summed device milliseconds, launches)."""
    ms = ctypes.c_float(0.0)
    n = ctypes.c_int32(0)
    _check("ls_kernel_timer_stop", lib().ls_kernel_timer_stop(ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)
