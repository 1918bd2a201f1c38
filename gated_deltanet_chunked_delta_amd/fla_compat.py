"""Drop-in entry with the calling convention of flash-linear-attention's
``chunk_gated_delta_rule`` (argument names, tensor layouts, return value), so
that a model written against that interface can take this package as its gated
DeltaNet backend without changing its call sites: the integration the "FlashQLA
resource" page describes in section 5 (entry signatures aligned with FLA's, the
kernels serving as FLA's GDN backend) and "Qwen's FlashQLA targets the expensive
bit of long-context AI" lists among its key findings.

Only argument conversion happens here; the computation is the autograd
function of this package, i.e. the HIP kernels behind ``include/gdn.h``:

* q, k [B, T, H, K] and v [B, T, H, V] share one dtype (bf16, or fp32 at
  K = V = 64); k, v and beta are cast to q's dtype and g to fp32 when they differ
  (the casts are differentiable, so gradients reach the caller's dtypes);
* g [B, T, H] is the log-space decay and beta [B, T, H] the write strength;
* ``head_first=True`` takes [B, H, T, *] inputs and returns o in that layout;
* ``cu_seqlens`` is a device tensor of any integer dtype with B = 1 (packed
  sequences); the library needs an int32 device copy and a host copy, so it is
  read back once per call (one device synchronisation);
* initial_state / the final state are [N, H, K, V] fp32 (h = S^T);
* ``use_qk_l2norm_in_kernel`` normalises q and k inside the kernels (and the
  backward returns gradients with respect to the raw q and k);
* the return value is always ``(o, final_state)``, final_state None unless
  ``output_final_state``.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import chunk_gated_delta_rule as _chunk
from .binding import GDNError

__all__ = ["chunk_gated_delta_rule"]


def chunk_gated_delta_rule(
    q: torch.Tensor,
    k: torch.Tensor,
    v: torch.Tensor,
    g: torch.Tensor,
    beta: torch.Tensor,
    scale: Optional[float] = None,
    initial_state: Optional[torch.Tensor] = None,
    output_final_state: bool = False,
    cu_seqlens: Optional[torch.Tensor] = None,
    head_first: bool = False,
    use_qk_l2norm_in_kernel: bool = False,
):
    """(o, final_state) of the gated delta rule; see the module docstring for
    the conventions.  Differentiable in q, k, v, g, beta and initial_state."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise GDNError("q, k, v must be 4-d ([B, T, H, D], or [B, H, T, D] with head_first)")
    if g.dim() != 3 or beta.dim() != 3:
        raise GDNError("g and beta must be 3-d ([B, T, H], or [B, H, T] with head_first)")
    if cu_seqlens is not None and q.shape[0] != 1:
        raise GDNError(f"cu_seqlens needs batch size 1 (packed sequences), got {q.shape[0]}")
    if head_first:
        q, k, v = (x.transpose(1, 2) for x in (q, k, v))
        g, beta = g.transpose(1, 2), beta.transpose(1, 2)
    dt = q.dtype
    q = q.contiguous()
    k, v, beta = (x.to(dt).contiguous() for x in (k, v, beta))
    g = g.to(torch.float32).contiguous()
    h0 = None if initial_state is None else initial_state.to(torch.float32).contiguous()
    cu = cu_host = None
    if cu_seqlens is not None:
        cu_host = cu_seqlens.detach().to("cpu", torch.int32)
        cu = cu_host.to(q.device)
    if scale is None:
        scale = k.shape[-1] ** -0.5
    o, hT = _chunk(q, k, v, g, beta, scale=scale, initial_state=h0, output_final_state=True,
                   cu_seqlens=cu, cu_seqlens_host=cu_host, qk_norm=bool(use_qk_l2norm_in_kernel))
    if head_first:
        o = o.transpose(1, 2)
    return o, (hT if output_final_state else None)
