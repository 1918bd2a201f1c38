"""ctypes binding of the fp64 token-recurrence oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Shapes follow the product API: q, k ``[B,T,H,Dk]``, v ``[B,T,H,Dv]``,
g, beta ``[B,T,H]``; with ``cu_seqlens`` (int, ``[N+1]``) B must be 1 and the
sequences are packed along T.  States h0/hT/dhT/dh0 are ``[N,H,Dk,Dv]`` and hold
h = S^T of the gated delta rule S_t = e^{g_t} S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
o_t = scale * S_t q_t.  Everything is computed in float64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("GDN_ORACLE_LIB")  # another build of the oracle (build.py --sanitize)
        if path:
            if not os.path.exists(path):
                raise FileNotFoundError(path)
        else:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(ctypes.c_double)
        I64 = ctypes.POINTER(ctypes.c_int64)
        lib.gdn_oracle_fwd.argtypes = [ctypes.c_int, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       P, P, P, P, P, P, ctypes.c_double, P, P]
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_bwd.argtypes = [ctypes.c_int, I64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       P, P, P, P, P, P, ctypes.c_double, P, P,
                                       P, P, P, P, P, P]
        lib.gdn_oracle_bwd.restype = ctypes.c_int
        lib.gdn_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle uses (set OMP_NUM_THREADS before first use to change)."""
    return _load().gdn_oracle_threads()


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _cu(shape, cu_seqlens):
    B, T = shape[0], shape[1]
    if cu_seqlens is None:
        return np.arange(B + 1, dtype=np.int64) * T
    if B != 1:
        raise ValueError("cu_seqlens requires B == 1")
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("bad cu_seqlens")
    return cu


def fwd(q, k, v, g, beta, scale, h0=None, cu_seqlens=None):
    """Return (o [B,T,H,Dv], hT [N,H,Dk,Dv]) in float64."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    cu = _cu(q.shape, cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((B, T, H, Dv))
    hT = np.zeros((N, H, Dk, Dv))
    rc = _load().gdn_oracle_fwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, Dk, Dv,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                float(scale), _ptr(o), _ptr(hT))
    if rc:
        raise MemoryError("oracle forward failed to allocate")
    return o, hT


def bwd(q, k, v, g, beta, scale, do, h0=None, dhT=None, cu_seqlens=None):
    """Return dict dq, dk, dv, dg, dbeta, dh0 (float64) for loss <do, o> + <dhT, hT>."""
    q, k, v, g, beta, h0, do, dhT = map(_f64, (q, k, v, g, beta, h0, do, dhT))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    cu = _cu(q.shape, cu_seqlens)
    N = len(cu) - 1
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dg=np.zeros_like(g), dbeta=np.zeros_like(beta), dh0=np.zeros((N, H, Dk, Dv)))
    rc = _load().gdn_oracle_bwd(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, Dk, Dv,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                float(scale), _ptr(do), _ptr(dhT),
                                _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]))
    if rc:
        raise MemoryError("oracle backward failed to allocate")
    return out
