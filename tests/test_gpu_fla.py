"""The FLA-convention entry (``fla_compat.chunk_gated_delta_rule``) on the GPU:
forward values and autograd gradients against the fp64 oracle, and layout /
dtype conversions against the direct call (the same kernels, so bitwise)."""
import numpy as np
import pytest

import gdn_inputs
from oracle import prep, ref
from tests.helpers import TOL, relerr, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def leaves(x, dev, head_first=False, g_dtype=None, beta_dtype=None):
    """Leaf tensors (requires_grad) of a GDNInputs in the dtypes given; with
    head_first, q, k, v, g, beta are contiguous in the [B, H, T, *] layout."""
    import torch
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    hf = (lambda a: np.swapaxes(a, 1, 2)) if head_first else (lambda a: a)
    mk = lambda a, d: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d).requires_grad_(True)
    out = dict(q=mk(hf(x.q), dt), k=mk(hf(x.k), dt), v=mk(hf(x.v), dt), g=mk(hf(x.g), g_dtype or torch.float32),
               beta=mk(hf(x.beta), beta_dtype or dt))
    out["h0"] = None if x.h0 is None else mk(x.h0, torch.float32)
    return out


def run(x, dev, head_first=False, cu_dtype=None, l2norm=False, **dtypes):
    """(o, hT, grads) through the FLA-convention entry, loss <do, o> + <dhT, hT>."""
    import torch
    from gated_deltanet_chunked_delta_amd.fla_compat import chunk_gated_delta_rule
    t = leaves(x, dev, head_first, **dtypes)
    args = [t["q"], t["k"], t["v"], t["g"], t["beta"]]
    cu = None
    if x.cu_seqlens is not None:
        cu = torch.from_numpy(np.asarray(x.cu_seqlens)).to(cu_dtype or torch.int64).to(dev)
    o, hT = chunk_gated_delta_rule(*args, scale=x.scale, initial_state=t["h0"], output_final_state=True,
                                   cu_seqlens=cu, head_first=head_first, use_qk_l2norm_in_kernel=l2norm)
    if head_first:
        B, T, H = x.q.shape[:3]
        assert tuple(o.shape) == (B, H, T, x.v.shape[-1])
        o = o.transpose(1, 2)
    do = torch.from_numpy(x.do).to(dev).to(o.dtype)
    loss = (o.float() * do.float()).sum()
    if x.dhT is not None:
        loss = loss + (hT * torch.from_numpy(x.dhT).to(dev)).sum()
    loss.backward()
    torch.cuda.synchronize()
    back = (lambda a: a.transpose(1, 2)) if head_first else (lambda a: a)
    grads = dict(dq=back(t["q"].grad), dk=back(t["k"].grad), dv=back(t["v"].grad), dg=back(t["g"].grad),
                 dbeta=back(t["beta"].grad), dh0=None if t["h0"] is None else t["h0"].grad)
    return o.detach(), hT.detach(), grads


def check_against_oracle(x, got, l2norm=False):
    o, hT, grads = got
    if l2norm:
        ro, rh = prep.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens, qk_norm=True)
        want = prep.bwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.do, x.h0, x.dhT, x.cu_seqlens, qk_norm=True)
    else:
        ro, rh = ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens)
        want = ref.bwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.do, x.h0, x.dhT, x.cu_seqlens)
    errs = {"o": relerr(to_np(o), ro), "hT": relerr(to_np(hT), rh)}
    for k, g in grads.items():
        if g is not None:
            errs[k] = relerr(to_np(g), want[k])
    print("    " + "  ".join(f"{k} {e:.3e}" for k, e in errs.items()), flush=True)
    bad = {k: e for k, e in errs.items() if not e <= TOL[x.dtype]}
    assert not bad, bad


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128)])
def test_fixed_length_matches_oracle(dev, Dk, Dv):
    print(f"[fla] fixed B=2 T=200 H=3 Dk={Dk} Dv={Dv}", flush=True)
    x = gdn_inputs.generate(2, 200, 3, Dk, Dv, "bf16", seed=71, h0_std=0.5, grad=True, dhT=True)
    check_against_oracle(x, run(x, dev))


def test_fp32_matches_oracle(dev):
    print("[fla] fp32 B=1 T=130 H=2", flush=True)
    x = gdn_inputs.generate(1, 130, 2, 64, 64, "f32", seed=72, h0_std=0.5, grad=True, dhT=True)
    check_against_oracle(x, run(x, dev))


@pytest.mark.parametrize("cu_dtype", ["int64", "int32"])
def test_packed_sequences(dev, cu_dtype):
    import torch
    print(f"[fla] varlen cu_seqlens {cu_dtype}", flush=True)
    x = gdn_inputs.generate(1, 0, 2, 64, 128, "bf16", seed=73, h0_std=0.5, lengths=(4, 1, 150), grad=True,
                            dhT=True)
    check_against_oracle(x, run(x, dev, cu_dtype=getattr(torch, cu_dtype)))


def test_head_first_layout_is_a_transpose(dev):
    print("[fla] head_first", flush=True)
    x = gdn_inputs.generate(2, 90, 3, 64, 64, "bf16", seed=74, h0_std=0.5, grad=True, dhT=True)
    a, b = run(x, dev), run(x, dev, head_first=True)
    assert torch_equal(a[0], b[0]) and torch_equal(a[1], b[1])
    for k in a[2]:
        assert torch_equal(a[2][k], b[2][k]), k


def test_l2norm_in_kernel(dev):
    print("[fla] use_qk_l2norm_in_kernel", flush=True)
    x = gdn_inputs.generate(1, 150, 2, 128, 128, "bf16", seed=75, h0_std=0.5, grad=True, dhT=True)
    # raw (unnormalised) q and k
    x.q = gdn_inputs.round_bf16(x.q * 3.0)
    x.k = gdn_inputs.round_bf16(x.k * 0.5)
    check_against_oracle(x, run(x, dev, l2norm=True), l2norm=True)


def test_dtype_casts_reach_the_caller(dev):
    import torch
    print("[fla] g in bf16, beta in fp32", flush=True)
    x = gdn_inputs.generate(1, 100, 2, 64, 64, "bf16", seed=76, h0_std=0.5, grad=True, dhT=True)
    x.g = gdn_inputs.round_bf16(x.g)  # representable in bf16, so both calls see the same g
    a = run(x, dev)
    b = run(x, dev, g_dtype=torch.bfloat16, beta_dtype=torch.float32)
    assert torch_equal(a[0], b[0]) and torch_equal(a[1], b[1])
    assert b[2]["dg"].dtype == torch.bfloat16 and b[2]["dbeta"].dtype == torch.float32
    for k in ("dq", "dk", "dv", "dh0"):
        assert torch_equal(a[2][k], b[2][k]), k
    assert torch_equal(a[2]["dg"].to(torch.bfloat16), b[2]["dg"])
    assert torch_equal(a[2]["dbeta"].float(), b[2]["dbeta"])


def test_final_state_only_when_asked(dev):
    import torch
    from gated_deltanet_chunked_delta_amd.fla_compat import chunk_gated_delta_rule
    x = gdn_inputs.generate(1, 64, 2, 64, 64, "bf16", seed=77)
    t = {k: torch.from_numpy(np.ascontiguousarray(getattr(x, k))).to(dev) for k in ("q", "k", "v", "g", "beta")}
    dt = torch.bfloat16
    o, hT = chunk_gated_delta_rule(t["q"].to(dt), t["k"].to(dt), t["v"].to(dt), t["g"].float(), t["beta"].to(dt))
    torch.cuda.synchronize()
    assert hT is None and tuple(o.shape) == (1, 64, 2, 64) and o.dtype == dt
    ro, _ = ref.fwd(x.q, x.k, x.v, x.g, x.beta, 64 ** -0.5)
    assert relerr(to_np(o), ro) <= TOL["bf16"]


def torch_equal(a, b):
    import torch
    return a.shape == b.shape and bool(torch.equal(a, b))
