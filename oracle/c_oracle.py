"""ctypes front end of the plain-C FP64 oracle (``gdn2_oracle.c``).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Same definition and
readings as :mod:`oracle.recurrence`; the pins in ``tests/test_oracle_pins.py``
run against both.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build_c_oracle
from .recurrence import l2_normalize_rows, resolve_scale

_F64, _F32, _BF16 = 0, 1, 2
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_c_oracle()  # a clean checkout: compile it (gcc, seconds)
        lib = ctypes.CDLL(LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.gdn2_oracle_fwd.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int,
                                        vp, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int,
                                        dbl, vp, ctypes.c_int, vp, i32, i64, i32, i32, i32, i32,
                                        vp, i32, vp, vp]
        lib.gdn2_oracle_fwd.restype = ctypes.c_int
        lib.gdn2_oracle_max_threads.restype = ctypes.c_int
        lib.gdn2_oracle_bwd.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int,
                                        vp, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int,
                                        dbl, vp, ctypes.c_int, vp, ctypes.c_int, vp, ctypes.c_int,
                                        vp, i32, i64, i32, i32, i32, i32, i32,
                                        vp, vp, vp, vp, vp, vp, vp]
        lib.gdn2_oracle_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _arr(x):
    """Return (contiguous numpy array, dtype code) with no precision change.

    Accepts numpy arrays (float64/float32) or torch CPU tensors (float64,
    float32, bfloat16 -- the latter passed as raw 16-bit patterns).
    """
    if x is None:
        return None, _F64
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), _BF16
            if x.dtype == torch.float32:
                return x.numpy(), _F32
            return x.to(torch.float64).numpy(), _F64
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a, _F32
    return np.ascontiguousarray(a, dtype=np.float64), _F64


load = _load


def max_threads() -> int:
    return int(_load().gdn2_oracle_max_threads())


def gdn2_recurrence_c(q, k, v, g=None, beta=None, w=None, scale=None,
                      initial_state=None, cu_seqlens=None, heads=None, qk_l2norm=False):
    """Same contract as :func:`oracle.recurrence.gdn2_recurrence` (with
    ``qk_l2norm`` the rows of q and k are normalised in float64 first, by the
    same reading, and the C loop runs on them)."""
    lib = _load()
    if qk_l2norm:
        q, k = l2_normalize_rows(q), l2_normalize_rows(k)
    qa, qd = _arr(q)
    ka, kd = _arr(k)
    va, vd = _arr(v)
    ga, gd = _arr(g)
    ba, bd = _arr(beta)
    wa, wd = _arr(w)
    sa, sd = _arr(initial_state)
    T, H, K = qa.shape
    HV, V = va.shape[1], va.shape[2]
    if cu_seqlens is None:
        cu = None
        N = 1
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).astype(np.int32))
        N = len(cu) - 1
    hv_idx = np.arange(HV, dtype=np.int32) if heads is None else np.asarray(heads, dtype=np.int32)
    hv_idx = np.ascontiguousarray(hv_idx)
    nh = len(hv_idx)
    out = np.zeros((T, nh, V), dtype=np.float64)
    final = np.zeros((N, nh, K, V), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.gdn2_oracle_fwd(ptr(qa), qd, ptr(ka), kd, ptr(va), vd, ptr(ga), gd,
                             ptr(ba), bd, ptr(wa), wd, resolve_scale(scale, K),
                             ptr(sa), sd, ptr(cu), N, T, H, HV, K, V,
                             hv_idx.ctypes.data, nh, out.ctypes.data, final.ctypes.data)
    if rc != 0:
        raise RuntimeError("C oracle rejected its arguments")
    return out, final


def gdn2_recurrence_bwd_c(q, k, v, g, beta, w, scale, initial_state, cu_seqlens, d_out,
                          d_final_state=None, block=64):
    """Same contract as :func:`oracle.recurrence_bwd.gdn2_recurrence_bwd`;
    ``block`` is the recompute block length of the C loop (it changes where
    states are recomputed, not the result)."""
    lib = _load()
    qa, qd = _arr(q)
    ka, kd = _arr(k)
    va, vd = _arr(v)
    ga, gd = _arr(g)
    ba, bd = _arr(beta)
    wa, wd = _arr(w)
    sa, sd = _arr(initial_state)
    da, dd = _arr(d_out)
    fa, fd = _arr(d_final_state)
    T, H, K = qa.shape
    HV, V = va.shape[1], va.shape[2]
    if cu_seqlens is None:
        cu, N = None, 1
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).astype(np.int32))
        N = len(cu) - 1
    dq = np.zeros((T, HV, K))
    dk = np.zeros((T, HV, K))
    dv = np.zeros((T, HV, V))
    dw = np.zeros((T, HV, V))
    dg = np.zeros((T, HV, K))
    db = np.zeros((T, HV, K))
    ds0 = np.zeros((N, HV, K, V))
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.gdn2_oracle_bwd(ptr(qa), qd, ptr(ka), kd, ptr(va), vd, ptr(ga), gd, ptr(ba), bd,
                             ptr(wa), wd, resolve_scale(scale, K), ptr(sa), sd, ptr(da), dd,
                             ptr(fa), fd, ptr(cu), N, T, H, HV, K, V, int(block),
                             dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, dw.ctypes.data,
                             dg.ctypes.data, db.ctypes.data, ds0.ctypes.data)
    if rc != 0:
        raise RuntimeError("C oracle rejected its arguments")
    m = HV // H
    return {"dq": dq.reshape(T, H, m, K).sum(axis=2), "dk": dk.reshape(T, H, m, K).sum(axis=2),
            "dv": dv, "dw": dw, "dg": dg, "dbeta": db, "d_initial_state": ds0}
