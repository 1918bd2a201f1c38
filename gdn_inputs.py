"""Seeded synthetic inputs for the chunked Gated DeltaNet prefill.

This module holds only random draws and dtype rounding -- none of the method's
arithmetic -- so that the fp64 oracle and the HIP path can be fed the same bits.
The pages ("FlashQLA resource", section 4) disclose no shapes or data for their
measurements, so these synthetic recipes are the workload itself.

Recipe (numpy ``Generator(PCG64(seed))``, float32 draws, in this order):
  lengths (varlen only, integers uniform on [lo, hi] inclusive),
  q, k ~ N(0,1) then scaled to unit L2 norm over the head dimension (per token, head),
  v ~ N(0,1),
  beta = sigmoid(N(0,1)),
  g = -softplus(N(0,1)) * 0.1     (natural-log decay, <= 0),
  h0 ~ h0_std * N(0,1)            (only when requested),
  do ~ N(0,1)                     (only when gradients are requested),
  dhT ~ N(0,1)                    (only when requested).
q, k, v, beta and do are then rounded to the compute dtype (bf16 with
round-to-nearest-even, or kept as fp32); g, h0 and dhT stay fp32.  Every array
is returned as float32 numpy holding exactly the values both sides consume.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


@dataclasses.dataclass
class GDNInputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    scale: float
    dtype: str                       # "f32" or "bf16"
    h0: Optional[np.ndarray] = None
    do: Optional[np.ndarray] = None
    dhT: Optional[np.ndarray] = None
    cu_seqlens: Optional[np.ndarray] = None   # int32 [N+1] or None

    @property
    def num_seqs(self) -> int:
        return self.q.shape[0] if self.cu_seqlens is None else len(self.cu_seqlens) - 1


def _unit(x: np.ndarray) -> np.ndarray:
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


def generate(B: int, T: int, H: int, Dk: int, Dv: int, dtype: str, seed: int,
             h0_std: Optional[float] = None, lengths: Optional[tuple] = None,
             grad: bool = False, dhT: bool = False) -> GDNInputs:
    """Draw one seeded input set.

    ``lengths=(N, lo, hi)`` makes a packed variable-length batch of N sequences
    (B must be 1, T is ignored and becomes the total length).
    """
    assert dtype in ("f32", "bf16")
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = None
    if lengths is not None:
        assert B == 1
        n, lo, hi = lengths
        L = rng.integers(lo, hi, size=n, endpoint=True)
        cu = np.zeros(n + 1, dtype=np.int32)
        cu[1:] = np.cumsum(L)
        T = int(cu[-1])
    nseq = B if cu is None else len(cu) - 1
    f = np.float32
    q = _unit(rng.standard_normal((B, T, H, Dk), dtype=f))
    k = _unit(rng.standard_normal((B, T, H, Dk), dtype=f))
    v = rng.standard_normal((B, T, H, Dv), dtype=f)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H), dtype=f).astype(np.float64)))).astype(f)
    z = rng.standard_normal((B, T, H), dtype=f).astype(np.float64)
    g = (-np.logaddexp(0.0, z) * 0.1).astype(f)
    h0 = None
    if h0_std is not None:
        h0 = (h0_std * rng.standard_normal((nseq, H, Dk, Dv), dtype=f)).astype(f)
    do = rng.standard_normal((B, T, H, Dv), dtype=f) if grad else None
    dht = rng.standard_normal((nseq, H, Dk, Dv), dtype=f) if dhT else None
    if dtype == "bf16":
        q, k, v, beta = (round_bf16(x) for x in (q, k, v, beta))
        if do is not None:
            do = round_bf16(do)
    return GDNInputs(q=q, k=k, v=v, g=g, beta=beta, scale=float(Dk) ** -0.5, dtype=dtype,
                     h0=h0, do=do, dhT=dht, cu_seqlens=cu)


# The five workloads the build is measured on, plus the long-sequence metric shape.
# name -> (kwargs for generate, seed)
CONFIGS = {
    "tiny_f32": dict(B=1, T=256, H=2, Dk=64, Dv=64, dtype="f32", seed=20260000),
    "single_bf16": dict(B=1, T=8192, H=16, Dk=128, Dv=128, dtype="bf16", seed=20260001, h0_std=0.02),
    "long_fewhead": dict(B=1, T=65536, H=4, Dk=128, Dv=128, dtype="bf16", seed=20260002),
    "varlen": dict(B=1, T=0, H=16, Dk=128, Dv=128, dtype="bf16", seed=20260003, lengths=(8, 512, 16384)),
    "train": dict(B=4, T=4096, H=16, Dk=128, Dv=128, dtype="bf16", seed=20260004, grad=True),
    "metric_32k": dict(B=1, T=32768, H=16, Dk=128, Dv=128, dtype="bf16", seed=20260005, grad=True),
}


def config(name: str, **override) -> GDNInputs:
    kw = dict(CONFIGS[name])
    kw.update(override)
    return generate(**kw)
