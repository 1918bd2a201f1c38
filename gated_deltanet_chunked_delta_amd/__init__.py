"""MI355X (gfx950) chunked Gated DeltaNet prefill: forward and backward.

The computation runs in hand-written HIP kernels behind the C ABI of
``include/gdn.h`` (``libgdn.so``); this package only marshals torch tensors
into it.  ``chunk_gated_delta_rule`` wraps the two entry points in an
autograd function.
"""
from __future__ import annotations

import torch

from .binding import GDNError, gdn_chunk_bwd, gdn_chunk_fwd, gdn_decode_step, lib  # noqa: F401

__all__ = ["gdn_chunk_fwd", "gdn_chunk_bwd", "gdn_decode_step", "chunk_gated_delta_rule", "GDNError", "lib"]


class _ChunkGatedDeltaRule(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, h0, scale, cu_seqlens, cu_seqlens_host, cp_mode, save_states,
                qk_norm, gate_act, gate_scale):
        res = gdn_chunk_fwd(q, k, v, g, beta, scale, h0=h0, cu_seqlens=cu_seqlens,
                            cu_seqlens_host=cu_seqlens_host, output_final_state=True, cp_mode=cp_mode,
                            save_states=save_states, save_t=True, qk_norm=qk_norm, gate_act=gate_act,
                            gate_scale=gate_scale)
        o, hT = res[0], res[1]
        states = res[2] if save_states else None
        chunk_t = res[-1]
        ctx.save_for_backward(q, k, v, g, beta, h0, cu_seqlens, states, chunk_t, gate_scale)
        ctx.scale, ctx.cu_host, ctx.cp_mode = scale, cu_seqlens_host, cp_mode
        ctx.qk_norm, ctx.gate_act = qk_norm, gate_act
        return o, hT

    @staticmethod
    def backward(ctx, do, dhT):
        q, k, v, g, beta, h0, cu, states, chunk_t, gate_scale = ctx.saved_tensors
        dq, dk, dv, dg, dbeta, dh0 = gdn_chunk_bwd(
            q, k, v, g, beta, ctx.scale, do.contiguous(), h0=h0,
            dhT=None if dhT is None else dhT.contiguous(), cu_seqlens=cu,
            cu_seqlens_host=ctx.cu_host, cp_mode=ctx.cp_mode, need_dh0=h0 is not None, states=states,
            chunk_t=chunk_t, qk_norm=ctx.qk_norm, gate_act=ctx.gate_act, gate_scale=gate_scale)
        return dq, dk, dv, dg, dbeta, dh0, None, None, None, None, None, None, None, None


def chunk_gated_delta_rule(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
                           cu_seqlens=None, cu_seqlens_host=None, cp_mode: int = 0, save_states: bool = True,
                           qk_norm: bool = False, gate_act: bool = False, gate_scale=None):
    """o, (hT) for the gated delta rule over [B, T, H, D] inputs, differentiable.

    g is the fp32 natural-log decay [B, T, H]; beta has the dtype of q.  The
    forward keeps every chunk's matrix T (64 x 64 fp32 per 64 tokens and head)
    for the backward.  With save_states (the default) it also keeps the state
    at every chunk start (Dk * Dv values per 64 tokens and head, in the input
    dtype) so that the backward does not recompute them; pass False to trade
    that memory for a forward replay inside the backward.  qk_norm: q and k are raw and normalised
    inside the kernels; gate_act: g and beta are logits, g = -gate_scale[h]
    softplus(g), beta = sigmoid(beta) inside the kernels (gate_scale is not
    differentiated).
    """
    if scale is None:
        scale = q.shape[-1] ** -0.5
    o, hT = _ChunkGatedDeltaRule.apply(q, k, v, g, beta, initial_state, float(scale), cu_seqlens,
                                       cu_seqlens_host, int(cp_mode), bool(save_states), bool(qk_norm),
                                       bool(gate_act), gate_scale)
    return (o, hT) if output_final_state else o
