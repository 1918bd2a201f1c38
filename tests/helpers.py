"""Shared test helpers: device transfer of seeded inputs and the error statistic."""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def relerr(gpu, ref):
    """max |gpu - ref| / max |ref| over one tensor (max |gpu - ref| if ref is all zero)."""
    a = np.asarray(gpu, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    den = np.abs(b).max()
    num = np.abs(a - b).max()
    return float(num / den) if den > 0 else float(num)


def to_torch(x, dev):
    """Device tensors of a gdn_inputs.GDNInputs in the dtypes the C ABI takes."""
    import torch
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    t = lambda a, d=dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d).contiguous()
    out = dict(q=t(x.q), k=t(x.k), v=t(x.v), beta=t(x.beta), g=t(x.g, torch.float32),
               h0=t(x.h0, torch.float32), do=t(x.do), dhT=t(x.dhT, torch.float32))
    out["cu"] = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(dev)
    return out


def to_np(t):
    return None if t is None else t.float().cpu().numpy()


def unblock_states(flat, C, H, Dk, Dv):
    """Chunk states as saved by gdn_chunk_fwd (flat, C * H * Dk * Dv elements; each
    state h, Dk x Dv, in 4 x 16 blocks as include/gdn.h states) -> numpy
    [C, H, Dk, Dv] holding h."""
    a = np.asarray(flat, dtype=np.float64)[:C * H * Dk * Dv]
    # [C, H, Dk/4, Dv/16, 4, 16] -> h[c, h, i, j] with i = 4 ib + ir, j = 16 jb + jr
    return a.reshape(C, H, Dk // 4, Dv // 16, 4, 16).transpose(0, 1, 2, 4, 3, 5).reshape(C, H, Dk, Dv)
