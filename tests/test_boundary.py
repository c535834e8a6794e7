"""The C ABI without a GPU: the library loads, exports every function include/ls_replay.h
declares, and rejects invalid arguments on the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from prefix_shared_branch_amd import lsreplay as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAD = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ls_\w+)\s*\(", src, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names == set(L.EXPORTED), names
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for c, s in ((0, "LS_OK"), (-1, "LS_ERR_INVALID_ARG"), (-2, "LS_ERR_UNSUPPORTED"), (-3, "LS_ERR_WORKSPACE"),
                 (-4, "LS_ERR_HIP"), (5, "LS_UNKNOWN_STATUS")):
        assert L.ls_status_string(c) == s


def desc(**kw):
    d = L.AttnDesc()
    d.P, d.Hq, d.Hkv, d.Dqk, d.Dv, d.ldk, d.ldv, d.softmax_scale = 1024, 8, 2, 64, 64, 128, 128, 0.125
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def ws_bytes(d, cu, which=0):
    cu = np.asarray(cu, dtype=np.int32)
    out = ctypes.c_size_t(0)
    rc = L.lib().ls_replay_attn_workspace_bytes(ctypes.byref(d), len(cu) - 1,
                                                cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), which,
                                                ctypes.byref(out))
    return rc, out.value


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=7), L.LS_ERR_INVALID_ARG),            # Hq % Hkv != 0
    (dict(P=-1), L.LS_ERR_INVALID_ARG),
    (dict(Hkv=0), L.LS_ERR_INVALID_ARG),
    (dict(Dqk=96, Dv=96, ldk=192, ldv=192), L.LS_ERR_UNSUPPORTED),
    (dict(Dv=128), L.LS_ERR_INVALID_ARG),           # Dv > Dqk
    (dict(ldk=120), L.LS_ERR_INVALID_ARG),          # ldk < Hkv * Dqk
    (dict(ldk=132), L.LS_ERR_INVALID_ARG),          # not a multiple of 8
    (dict(softmax_scale=float("nan")), L.LS_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), L.LS_ERR_INVALID_ARG),
])
def test_desc_validation(kw, code):
    assert ws_bytes(desc(**kw), [0, 100])[0] == code


def test_seqlens_validation():
    d = desc()
    assert ws_bytes(d, [1, 100])[0] == L.LS_ERR_INVALID_ARG         # cu[0] != 0
    assert ws_bytes(d, [0, 100, 50])[0] == L.LS_ERR_INVALID_ARG     # decreasing
    assert ws_bytes(d, list(range(0, 66)))[0] == L.LS_ERR_UNSUPPORTED  # 65 responses
    assert ws_bytes(d, [0, 0, 10])[0] == L.LS_OK                    # empty response allowed
    assert ws_bytes(d, [0, 100], which=3)[0] == L.LS_ERR_INVALID_ARG
    rc, n = ws_bytes(desc(P=0), [0, 10], which=1)
    assert rc == L.LS_OK and n > 0                                   # delta buffer


def _fwd(d, cu, Kp=BAD, Vp=BAD, Q=BAD, Ks=BAD, Vs=BAD, O=BAD, lse=BAD, O_lo=None, ws=BAD, nbytes=1 << 40):
    cu = np.asarray(cu, dtype=np.int32)
    return L.lib().ls_replay_attn_fwd(None, ctypes.byref(d), Kp, Vp, len(cu) - 1,
                                      cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), Q, Ks, Vs, O, lse, O_lo, ws,
                                      nbytes)


def _bwd(d, cu, dKp=BAD, dVp=BAD, ws=BAD, nbytes=1 << 40, Q=BAD, O_lo=None):
    cu = np.asarray(cu, dtype=np.int32)
    return L.lib().ls_replay_attn_bwd(None, ctypes.byref(d), BAD, BAD, len(cu) - 1,
                                      cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), Q, BAD, BAD, BAD, BAD,
                                      O_lo, BAD, BAD, BAD, BAD, dKp, dVp, ws, nbytes)


def test_fwd_bwd_pointer_and_workspace_validation():
    d = desc()
    assert _fwd(d, [0, 10], Q=None) == L.LS_ERR_INVALID_ARG
    assert _fwd(d, [0, 10], Q=ctypes.c_void_p(0x1008)) == L.LS_ERR_INVALID_ARG   # misaligned
    assert _fwd(d, [0, 10], Kp=None) == L.LS_ERR_INVALID_ARG                     # P > 0 needs prompt K
    assert _fwd(d, [0, 0]) == L.LS_OK                                            # nothing to do
    rc, need = ws_bytes(desc(P=1 << 20), [0, 64], 0)
    assert rc == L.LS_OK and need > 0
    assert _fwd(desc(P=1 << 20), [0, 64], nbytes=need - 1) == L.LS_ERR_WORKSPACE
    assert _fwd(desc(P=1 << 20), [0, 64], ws=None, nbytes=need) == L.LS_ERR_WORKSPACE
    assert _bwd(d, [0, 10], dKp=None) == L.LS_ERR_INVALID_ARG                    # exactly one accumulator
    assert _bwd(d, [0, 10], dVp=None) == L.LS_ERR_INVALID_ARG
    assert _bwd(d, [0, 10], dKp=None, dVp=None, Q=None) == L.LS_ERR_INVALID_ARG
    assert _bwd(d, [0, 10], nbytes=0) == L.LS_ERR_WORKSPACE
    # the optional rounding residual of O: NULL is accepted, a misaligned pointer is not
    assert _fwd(d, [0, 10], O_lo=ctypes.c_void_p(0x1008)) == L.LS_ERR_INVALID_ARG
    assert _bwd(d, [0, 10], O_lo=ctypes.c_void_p(0x1008)) == L.LS_ERR_INVALID_ARG


def _block_ws(d, q0, nq, which=0):
    n = ctypes.c_size_t(0)
    return L.lib().ls_replay_attn_block_workspace_bytes(ctypes.byref(d), q0, nq, which, ctypes.byref(n)), n.value


def _fwd_block(d, q0, nq, Q=BAD, Ks=BAD, ws=BAD, nbytes=1 << 40):
    return L.lib().ls_replay_attn_fwd_block(None, ctypes.byref(d), BAD, BAD, q0, nq, Q, Ks, BAD, BAD, BAD, None, ws,
                                            nbytes)


def _bwd_block(d, q0, nq, dKs=BAD, dVs=BAD, dKp=BAD, dVp=BAD, ws=BAD, nbytes=1 << 40):
    return L.lib().ls_replay_attn_bwd_block(None, ctypes.byref(d), BAD, BAD, q0, nq, BAD, BAD, BAD, BAD, BAD, None,
                                            BAD, BAD, dKs, dVs, dKp, dVp, ws, nbytes)


def test_block_validation():
    d = desc()
    assert _block_ws(d, -1, 10)[0] == L.LS_ERR_INVALID_ARG
    assert _block_ws(d, 0, -1)[0] == L.LS_ERR_INVALID_ARG
    assert _block_ws(d, 0, 10, which=3)[0] == L.LS_ERR_INVALID_ARG
    rc0, n0 = _block_ws(d, 0, 100)
    rc1, n1 = _block_ws(d, 900, 100)
    assert rc0 == L.LS_OK and rc1 == L.LS_OK and n1 > n0    # the block's earlier keys are packed too
    assert _block_ws(desc(Dqk=96, Dv=96, ldk=192, ldv=192), 0, 10)[0] == L.LS_ERR_UNSUPPORTED
    assert _fwd_block(d, -5, 10) == L.LS_ERR_INVALID_ARG
    assert _fwd_block(d, 5, 10, Q=None) == L.LS_ERR_INVALID_ARG
    assert _fwd_block(d, 5, 10, Ks=ctypes.c_void_p(0x1008)) == L.LS_ERR_INVALID_ARG  # misaligned
    assert _fwd_block(d, 5, 0) == L.LS_OK                                           # nothing to do
    assert _bwd_block(d, 5, 10, dKs=None) == L.LS_ERR_INVALID_ARG                   # key accumulators required
    assert _bwd_block(d, 5, 10, dVs=None) == L.LS_ERR_INVALID_ARG
    assert _bwd_block(d, 5, 10, dKp=None) == L.LS_ERR_INVALID_ARG                   # exactly one prompt accumulator
    assert _bwd_block(d, 5, 10, nbytes=0) == L.LS_ERR_WORKSPACE


def _loss(V=4096, G=2, R=(3, 4), rewards=(0.0, 1.0), eps=0.2, first=0, count=2, logits=BAD, dl=ctypes.c_void_p(0x90000),
          ws=BAD, nbytes=1 << 30, targets=BAD):
    Ra = np.asarray(R, dtype=np.int32)
    ra = np.asarray(rewards, dtype=np.float32)
    return L.lib().ls_grpo_token_loss(None, V, G, Ra.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      ra.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), eps, first, count, logits,
                                      targets, BAD, dl, BAD, None, None, ws, nbytes)


def test_loss_validation():
    assert _loss(V=0) == L.LS_ERR_INVALID_ARG
    assert _loss(V=(1 << 24) + 8) == L.LS_ERR_UNSUPPORTED           # beyond 32-bit element offsets
    assert _loss(eps=0.0) == L.LS_ERR_INVALID_ARG
    assert _loss(eps=1.0) == L.LS_ERR_INVALID_ARG
    assert _loss(eps=float("nan")) == L.LS_ERR_INVALID_ARG
    assert _loss(R=(0, 4)) == L.LS_ERR_INVALID_ARG                  # R_i <= 0
    assert _loss(rewards=(0.0, float("inf"))) == L.LS_ERR_INVALID_ARG
    assert _loss(first=1, count=2) == L.LS_ERR_INVALID_ARG          # beyond G
    assert _loss(count=0) == L.LS_ERR_INVALID_ARG
    assert _loss(targets=None) == L.LS_ERR_INVALID_ARG
    assert _loss(dl=BAD) == L.LS_ERR_INVALID_ARG                    # dlogits aliases logits
    assert _loss(ws=None) == L.LS_ERR_WORKSPACE
    assert _loss(nbytes=4) == L.LS_ERR_WORKSPACE
    out = ctypes.c_size_t(0)
    assert L.lib().ls_grpo_workspace_bytes(1000, 4096, ctypes.byref(out)) == L.LS_OK and out.value >= 4000
    assert L.lib().ls_grpo_workspace_bytes(-1, 4096, ctypes.byref(out)) == L.LS_ERR_INVALID_ARG


def test_kernel_timer_validation():
    lib = L.lib()
    ms, n = ctypes.c_float(1.0), ctypes.c_int32(7)
    # stop without start: invalid, outputs cleared, no HIP call made
    assert lib.ls_kernel_timer_stop(ctypes.byref(ms), ctypes.byref(n)) == L.LS_ERR_INVALID_ARG
    assert ms.value == 0.0 and n.value == 0
    for bad in (-1, 4, 100):
        assert lib.ls_kernel_timer_start(bad) == L.LS_ERR_INVALID_ARG
    assert lib.ls_kernel_timer_stop(None, None) == L.LS_ERR_INVALID_ARG
    # armed, nothing launched: zero launches and zero time, without touching the device
    assert lib.ls_kernel_timer_start(L.LS_KERNEL_DQ) == L.LS_OK
    assert lib.ls_kernel_timer_stop(ctypes.byref(ms), ctypes.byref(n)) == L.LS_OK
    assert ms.value == 0.0 and n.value == 0


def _latent(**kw):
    base = dict(P=4096, Hq=16, Hkv=1, Dqk=576, Dv=512, ldk=576, ldv=576, softmax_scale=1.0 / 24.0)
    base.update(kw)
    return desc(**base)


def test_latent_kv_shape_validation():
    """(576, 512) heads are served only as latent KV: one kv head, V rows = the K rows' leading dims."""
    for which in (0, 1, 2):
        rc, n = ws_bytes(_latent(), [0, 100, 300], which)
        assert rc == L.LS_OK and n > 0
    assert ws_bytes(_latent(Hq=32, Hkv=2, ldk=1152, ldv=1152), [0, 10])[0] == L.LS_ERR_UNSUPPORTED
    assert ws_bytes(_latent(ldv=512), [0, 10])[0] == L.LS_ERR_UNSUPPORTED
    assert ws_bytes(_latent(Dv=448, ldv=576), [0, 10])[0] == L.LS_ERR_UNSUPPORTED
    assert _block_ws(_latent(), 100, 50, 1)[0] == L.LS_OK


def test_latent_kv_requires_aliased_v():
    d = _latent()
    K, V = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    # checked before any device work: a separate V buffer is refused, the aliased form passes
    assert _fwd(d, [0, 0], Kp=K, Vp=V, Ks=K, Vs=K) == L.LS_ERR_UNSUPPORTED
    assert _fwd(d, [0, 0], Kp=K, Vp=K, Ks=K, Vs=V) == L.LS_ERR_UNSUPPORTED
    assert _fwd(d, [0, 0], Kp=K, Vp=K, Ks=V, Vs=V) == L.LS_OK
    assert _fwd(_latent(P=0), [0, 0], Kp=None, Vp=None, Ks=V, Vs=V) == L.LS_OK


def _lm(V=4096, d=256, G=2, R=(3, 4), first=0, count=2, H=BAD, W=BAD, dH=BAD, dW=BAD, ws=BAD, nbytes=1 << 40,
        eps=0.2):
    Ra = np.asarray(R, dtype=np.int32)
    rw = np.asarray([1.0, 0.0][:len(R)] + [0.0] * max(0, len(R) - 2), dtype=np.float32)
    return L.lib().ls_grpo_lmhead_loss(None, V, d, G, Ra.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                       rw.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), eps, first, count, H, W,
                                       BAD, BAD, BAD, dH, dW, None, None, ws, nbytes)


def test_lmhead_validation():
    """Argument checks of the LM-head entry point, all before any device work."""
    n = ctypes.c_size_t(0)
    assert L.lib().ls_grpo_lmhead_workspace_bytes(5000, 4096, 256, ctypes.byref(n)) == L.LS_OK
    assert n.value >= 2 * 2048 * 4096 * 2                       # logits and dlogits of one chunk
    assert L.lib().ls_grpo_lmhead_workspace_bytes(-1, 4096, 256, ctypes.byref(n)) == L.LS_ERR_INVALID_ARG
    assert _lm(V=4100) == L.LS_ERR_UNSUPPORTED                   # rows of the loss kernel: V % 8 == 0
    assert _lm(d=250) == L.LS_ERR_UNSUPPORTED
    assert _lm(V=(1 << 24) + 8) == L.LS_ERR_UNSUPPORTED
    assert _lm(dH=None) == L.LS_ERR_INVALID_ARG                  # gradients come in pairs
    assert _lm(dW=None) == L.LS_ERR_INVALID_ARG
    assert _lm(H=None) == L.LS_ERR_INVALID_ARG
    assert _lm(H=ctypes.c_void_p(0x1008)) == L.LS_ERR_INVALID_ARG   # misaligned
    assert _lm(first=1, count=2) == L.LS_ERR_INVALID_ARG
    assert _lm(eps=1.5) == L.LS_ERR_INVALID_ARG
    assert _lm(R=(3, 0)) == L.LS_ERR_INVALID_ARG
    assert _lm(nbytes=100) == L.LS_ERR_WORKSPACE
    assert _lm(ws=None) == L.LS_ERR_WORKSPACE
