"""fp64 oracle of the optional input pre-processing, composed with the token
recurrence of ``ref``.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The operator's inputs are usually produced from raw projections: q and k are
L2-normalised per (token, head) vector and the gate and the write strength come
from logits ("FlashQLA resource", section 3, lists fusing such surrounding work
into the kernels among its techniques).  The definitions used here:

    q_hat = q / sqrt(|q|^2 + 1e-6),   k_hat likewise (over the head dimension)
    g     = -gate_scale[h] * softplus(a),        beta = sigmoid(b)

and the operator is the gated delta rule of ``ref`` applied to
(q_hat, k_hat, v, g, beta).  The backward is the chain rule through these
maps:

    dq = (dq_hat - q_hat (q_hat . dq_hat)) / sqrt(|q|^2 + 1e-6)   (k likewise)
    da = -gate_scale[h] * sigmoid(a) * dg,    db = beta (1 - beta) * dbeta

Everything in float64.
"""
import numpy as np

from . import ref

EPS = 1e-6


def _norm(x):
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)
    return x / n, n


def _softplus(a):
    return np.logaddexp(0.0, a)


def _sigmoid(b):
    return 0.5 * (1.0 + np.tanh(0.5 * b))


def inputs(q, k, g, beta, qk_norm=False, gate_act=False, gate_scale=None):
    """The kernel inputs (q, k, g, beta) after the pre-processing, in float64."""
    q, k, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, g, beta))
    if qk_norm:
        q, _ = _norm(q)
        k, _ = _norm(k)
    if gate_act:
        s = np.ones(g.shape[-1]) if gate_scale is None else np.asarray(gate_scale, dtype=np.float64)
        g = -s * _softplus(g)
        beta = _sigmoid(beta)
    return q, k, g, beta


def fwd(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, qk_norm=False, gate_act=False, gate_scale=None):
    """(o, hT) of the gated delta rule on the pre-processed inputs."""
    qh, kh, gg, bb = inputs(q, k, g, beta, qk_norm, gate_act, gate_scale)
    return ref.fwd(qh, kh, v, gg, bb, scale, h0, cu_seqlens)


def bwd(q, k, v, g, beta, scale, do, h0=None, dhT=None, cu_seqlens=None, qk_norm=False, gate_act=False,
        gate_scale=None):
    """Gradients with respect to the raw inputs (dict as ``ref.bwd``)."""
    qh, kh, gg, bb = inputs(q, k, g, beta, qk_norm, gate_act, gate_scale)
    out = ref.bwd(qh, kh, v, gg, bb, scale, do, h0, dhT, cu_seqlens)
    if qk_norm:
        for name, raw in (("dq", q), ("dk", k)):
            xh, n = _norm(raw)
            d = out[name]
            out[name] = (d - xh * np.sum(xh * d, axis=-1, keepdims=True)) / n
    if gate_act:
        a = np.asarray(g, dtype=np.float64)
        s = np.ones(a.shape[-1]) if gate_scale is None else np.asarray(gate_scale, dtype=np.float64)
        out["dg"] = -s * _sigmoid(a) * out["dg"]
        out["dbeta"] = bb * (1.0 - bb) * out["dbeta"]
    return out
