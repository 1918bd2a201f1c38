"""ctypes binding of ``libgdn.so`` (the C ABI in ``include/gdn.h``).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  There is
no fallback -- if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB selects another build of the same library (for instance one whose host
# code carries sanitizers, see build.py --sanitize); there is no other fallback.
LIB_PATH = os.environ.get("GDN_LIB") or os.path.join(HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_E_INVALID", 2: "GDN_E_UNSUPPORTED", 3: "GDN_E_WORKSPACE", 4: "GDN_E_HIP"}

_vp = ctypes.c_void_p


class CommonArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("T", ctypes.c_int32),
                ("H", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("g", _vp), ("beta", _vp), ("h0", _vp),
                ("scale", ctypes.c_float),
                ("cu_seqlens", _vp), ("cu_seqlens_host", _vp),
                ("num_seqs", ctypes.c_int32), ("cp_mode", ctypes.c_int32),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("qk_norm", ctypes.c_int32), ("gate_act", ctypes.c_int32), ("gate_scale", _vp)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("a", CommonArgs), ("o", _vp), ("hT", _vp), ("h_save", _vp), ("t_save", _vp)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("a", CommonArgs), ("h_saved", _vp), ("t_saved", _vp), ("do_", _vp), ("dhT", _vp), ("dq", _vp),
                ("dk", _vp),
                ("dv", _vp), ("dbeta", _vp), ("dg", _vp), ("dh0", _vp)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("N", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("g", _vp), ("beta", _vp),
                ("scale", ctypes.c_float), ("state", _vp), ("state_idx", _vp),
                ("num_slots", ctypes.c_int32), ("o", _vp),
                ("qk_norm", ctypes.c_int32), ("gate_act", ctypes.c_int32), ("gate_scale", _vp)]


class GDNError(RuntimeError):
    pass


_lib = None


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GDNError(f"{LIB_PATH} is missing: build it with gated_deltanet_chunked_delta_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdArgs)]
        L.gdn_chunk_fwd_workspace_size.restype = ctypes.c_size_t
        L.gdn_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
        L.gdn_chunk_bwd_workspace_size.restype = ctypes.c_size_t
        L.gdn_chunk_states_bytes.argtypes = [ctypes.POINTER(CommonArgs)]
        L.gdn_chunk_states_bytes.restype = ctypes.c_size_t
        L.gdn_chunk_t_bytes.argtypes = [ctypes.POINTER(CommonArgs)]
        L.gdn_chunk_t_bytes.restype = ctypes.c_size_t
        L.gdn_chunk_fwd.argtypes = [ctypes.POINTER(FwdArgs), _vp]
        L.gdn_chunk_fwd.restype = ctypes.c_int
        L.gdn_chunk_bwd.argtypes = [ctypes.POINTER(BwdArgs), _vp]
        L.gdn_chunk_bwd.restype = ctypes.c_int
        L.gdn_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(FwdArgs), _vp]
        L.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
        L.gdn_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        L.gdn_decode_step.restype = ctypes.c_int
        L.gdn_profile_enable.argtypes = [ctypes.c_int]
        L.gdn_profile_enable.restype = ctypes.c_int
        L.gdn_profile_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
        L.gdn_profile_read.restype = ctypes.c_int
        L.gdn_profile_reset.restype = None
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        msg = lib().gdn_last_error().decode()
        raise GDNError(f"{STATUS.get(status, status)}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise GDNError(f"unsupported dtype {t.dtype}")


def _contig(name, t, dtype=None, device=None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise GDNError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GDNError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise GDNError(f"{name} must be on {device}")
    return t


def _prep(a, q, qk_norm, gate_act, gate_scale):
    """Fill the pre-processing fields of an argument struct."""
    a.qk_norm, a.gate_act = int(bool(qk_norm)), int(bool(gate_act))
    if gate_scale is not None:
        _contig("gate_scale", gate_scale, torch.float32, q.device)
        if gate_scale.numel() != a.H:
            raise GDNError("gate_scale must have H entries")
    a.gate_scale = _ptr(gate_scale)


def _common(q, k, v, g, beta, scale, h0, cu_seqlens, cu_seqlens_host, cp_mode,
            qk_norm=False, gate_act=False, gate_scale=None):
    dev = q.device
    dt = q.dtype
    _contig("q", q, dt, dev)
    _contig("k", k, dt, dev)
    _contig("v", v, dt, dev)
    _contig("beta", beta, dt, dev)
    _contig("g", g, torch.float32, dev)
    _contig("h0", h0, torch.float32, dev)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (B, T, H, Dk) or tuple(v.shape[:3]) != (B, T, H):
        raise GDNError("q, k, v shapes disagree")
    if tuple(g.shape) != (B, T, H) or tuple(beta.shape) != (B, T, H):
        raise GDNError("g and beta must be [B, T, H]")
    a = CommonArgs()
    a.dtype = _dtype_code(q)
    a.B, a.T, a.H, a.Dk, a.Dv = B, T, H, Dk, Dv
    a.q, a.k, a.v, a.g, a.beta, a.h0 = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0)
    a.scale = float(scale)
    keep = []
    if cu_seqlens is not None:
        _contig("cu_seqlens", cu_seqlens, torch.int32, dev)
        if cu_seqlens_host is None:
            cu_seqlens_host = cu_seqlens.cpu()  # synchronises; pass the host copy to avoid it
        host = torch.as_tensor(cu_seqlens_host, dtype=torch.int32).contiguous()
        keep.append(host)
        a.cu_seqlens = cu_seqlens.data_ptr()
        a.cu_seqlens_host = host.data_ptr()
        a.num_seqs = host.numel() - 1
    else:
        a.num_seqs = B
    a.cp_mode = int(cp_mode)
    _prep(a, q, qk_norm, gate_act, gate_scale)
    return a, keep


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def gdn_chunk_fwd(q, k, v, g, beta, scale: float, h0=None, cu_seqlens=None, cu_seqlens_host=None,
                  output_final_state: bool = True, cp_mode: int = 0, save_states: bool = False,
                  save_t: bool = False, qk_norm: bool = False, gate_act: bool = False, gate_scale=None,
                  o=None, hT=None, noalloc: bool = False):
    """Forward pass.  Returns (o, hT) with hT None unless output_final_state, followed by
    states if save_states (the state at every chunk start, a flat tensor of the input
    dtype) and chunk_t if save_t (every chunk's matrix T, a flat fp32 tensor laid out as
    gdn_chunk_t_bytes in include/gdn.h describes); both are
    for gdn_chunk_bwd.  qk_norm / gate_act select the in-kernel pre-processing (raw q,
    k; gate and beta logits, see include/gdn.h).  o / hT: optional output tensors
    to write into (else allocated).  noalloc: call gdn_chunk_fwd_noalloc, which
    takes no workspace (the library's own scratch; see include/gdn.h)."""
    a, keep = _common(q, k, v, g, beta, scale, h0, cu_seqlens, cu_seqlens_host, cp_mode,
                      qk_norm, gate_act, gate_scale)
    L = lib()
    if o is None:
        o = torch.empty(q.shape[:3] + (a.Dv,), dtype=q.dtype, device=q.device)
    _contig("o", o, q.dtype, q.device)
    if tuple(o.shape) != tuple(q.shape[:3]) + (a.Dv,):
        raise GDNError("o has the wrong shape")
    if hT is None and output_final_state:
        hT = torch.empty((a.num_seqs, a.H, a.Dk, a.Dv), dtype=torch.float32, device=q.device)
    if hT is not None:
        _contig("hT", hT, torch.float32, q.device)
        if tuple(hT.shape) != (a.num_seqs, a.H, a.Dk, a.Dv):
            raise GDNError("hT has the wrong shape")
    states = None
    if save_states:
        nb = L.gdn_chunk_states_bytes(ctypes.byref(a))
        states = torch.empty(max(nb, 16) // q.element_size(), dtype=q.dtype, device=q.device)
    chunk_t = None
    if save_t:
        nb = L.gdn_chunk_t_bytes(ctypes.byref(a))
        chunk_t = torch.empty(max(nb, 16) // 4, dtype=torch.float32, device=q.device)
    args = FwdArgs()
    args.a = a
    args.o, args.hT, args.h_save, args.t_save = _ptr(o), _ptr(hT), _ptr(states), _ptr(chunk_t)
    if noalloc:
        _check(L.gdn_chunk_fwd_noalloc(ctypes.byref(args), _vp(_stream(q.device))))
        del keep
        return (o, hT) + ((states,) if save_states else ()) + ((chunk_t,) if save_t else ())
    nbytes = L.gdn_chunk_fwd_workspace_size(ctypes.byref(args))
    if nbytes == 0:
        _check(1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    args.a.workspace, args.a.workspace_bytes = ws.data_ptr(), nbytes
    _check(L.gdn_chunk_fwd(ctypes.byref(args), _vp(_stream(q.device))))
    del keep
    return (o, hT) + ((states,) if save_states else ()) + ((chunk_t,) if save_t else ())


def gdn_chunk_bwd(q, k, v, g, beta, scale: float, do, h0=None, dhT=None, cu_seqlens=None,
                  cu_seqlens_host=None, cp_mode: int = 0, need_dh0: bool = True, states=None,
                  chunk_t=None, qk_norm: bool = False, gate_act: bool = False, gate_scale=None):
    """Backward pass.  Returns (dq, dk, dv, dg, dbeta, dh0) with dh0 None unless need_dh0.
    states / chunk_t: the forward's saved chunk states and chunk matrices T
    (gdn_chunk_fwd(..., save_states=True / save_t=True)); what is given is not
    recomputed.  With qk_norm / gate_act the gradients are with respect to the raw
    inputs."""
    a, keep = _common(q, k, v, g, beta, scale, h0, cu_seqlens, cu_seqlens_host, cp_mode,
                      qk_norm, gate_act, gate_scale)
    _contig("do", do, q.dtype, q.device)
    _contig("dhT", dhT, torch.float32, q.device)
    _contig("states", states, q.dtype, q.device)
    if states is not None and states.numel() * states.element_size() < lib().gdn_chunk_states_bytes(ctypes.byref(a)):
        raise GDNError("states is smaller than gdn_chunk_states_bytes")
    _contig("chunk_t", chunk_t, torch.float32, q.device)
    if chunk_t is not None and chunk_t.numel() * 4 < lib().gdn_chunk_t_bytes(ctypes.byref(a)):
        raise GDNError("chunk_t is smaller than gdn_chunk_t_bytes")
    L = lib()
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv = torch.empty_like(v)
    dbeta = torch.empty_like(beta)
    dg = torch.empty_like(g)
    dh0 = (torch.empty((a.num_seqs, a.H, a.Dk, a.Dv), dtype=torch.float32, device=q.device)
           if need_dh0 else None)
    args = BwdArgs()
    args.a = a
    args.h_saved, args.t_saved = _ptr(states), _ptr(chunk_t)
    args.do_, args.dhT = _ptr(do), _ptr(dhT)
    args.dq, args.dk, args.dv, args.dbeta, args.dg, args.dh0 = map(_ptr, (dq, dk, dv, dbeta, dg, dh0))
    nbytes = L.gdn_chunk_bwd_workspace_size(ctypes.byref(args))
    if nbytes == 0:
        _check(1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    args.a.workspace, args.a.workspace_bytes = ws.data_ptr(), nbytes
    _check(L.gdn_chunk_bwd(ctypes.byref(args), _vp(_stream(q.device))))
    del keep
    return dq, dk, dv, dg, dbeta, dh0


def gdn_decode_step(q, k, v, g, beta, scale: float, state, state_idx=None, o=None,
                    qk_norm: bool = False, gate_act: bool = False, gate_scale=None):
    """One recurrent step for N sequences: q, k [N, H, Dk], v [N, H, Dv], g, beta [N, H];
    state [S, H, Dk, Dv] fp32 is updated in place (sequence n uses slot n, or state_idx[n]
    when given; out-of-range indices mark padding).  Returns o [N, H, Dv]."""
    dev = q.device
    dt = q.dtype
    for name, t, d in (("q", q, dt), ("k", k, dt), ("v", v, dt), ("beta", beta, dt),
                       ("g", g, torch.float32), ("state", state, torch.float32)):
        _contig(name, t, d, dev)
    _contig("state_idx", state_idx, torch.int32, dev)
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    if tuple(k.shape) != (N, H, Dk) or tuple(v.shape[:2]) != (N, H) or tuple(g.shape) != (N, H) \
            or tuple(beta.shape) != (N, H) or tuple(state.shape[1:]) != (H, Dk, Dv):
        raise GDNError("decode shapes disagree")
    if o is None:
        o = torch.empty((N, H, Dv), dtype=dt, device=dev)
    a = DecodeArgs()
    a.dtype, a.N, a.H, a.Dk, a.Dv = _dtype_code(q), N, H, Dk, Dv
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.scale = float(scale)
    a.state, a.state_idx, a.num_slots, a.o = _ptr(state), _ptr(state_idx), state.shape[0], _ptr(o)
    _prep(a, q, qk_norm, gate_act, gate_scale)
    _check(lib().gdn_decode_step(ctypes.byref(a), _vp(_stream(dev))))
    return o


def gdn_profile_enable(on: bool) -> bool:
    """Turn per-kernel event timing on or off; returns the previous setting."""
    return bool(lib().gdn_profile_enable(1 if on else 0))


def gdn_profile_reset() -> None:
    lib().gdn_profile_reset()


def gdn_profile_read() -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset (waits for the events)."""
    L = lib()
    cap = 32
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int * cap)()
    n = L.gdn_profile_read(cap, names, ms, cnt)
    if n < 0:
        _check(4)
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n, cap))}


def exported_symbols(header: Optional[str] = None) -> Sequence[str]:
    """Function names declared in include/gdn.h."""
    import re
    header = header or os.path.join(os.path.dirname(HERE), "include", "gdn.h")
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))
