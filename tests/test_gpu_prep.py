"""In-kernel pre-processing on the GPU (raw q, k normalised inside the kernels;
gate and beta from logits): forward, backward and decode through the C ABI
against the fp64 oracle of the composed operator, element by element."""
import numpy as np
import pytest

import gdn_inputs
from gdn_inputs import round_bf16
from oracle import prep
from tests.helpers import TOL, relerr, to_np, to_torch

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def make_raw(x, seed):
    """Raw inputs around a generated workload: every q / k vector scaled by its own
    factor in [0.25, 4], gate and beta logits ~ N(0, 1) (beta logits in the input
    dtype), and a per-head gate scale of 0.1."""
    rng = np.random.default_rng(seed)
    rnd = round_bf16 if x.dtype == "bf16" else (lambda a: a.astype(np.float32))
    x.q = rnd(x.q * rng.uniform(0.25, 4.0, size=x.q.shape[:-1] + (1,)))
    x.k = rnd(x.k * rng.uniform(0.25, 4.0, size=x.k.shape[:-1] + (1,)))
    x.g = rng.standard_normal(x.g.shape).astype(np.float32)
    x.beta = rnd(rng.standard_normal(x.beta.shape))
    gate_scale = np.full(x.q.shape[2], 0.1, dtype=np.float32)
    return x, gate_scale


def kw_torch(gs, dev):
    import torch
    return dict(qk_norm=True, gate_act=True, gate_scale=torch.from_numpy(gs).to(dev))


@pytest.mark.parametrize("dtype,Dk,Dv,T,cp", [("bf16", 128, 128, 200, 0), ("bf16", 128, 128, 700, 3),
                                             ("bf16", 64, 128, 130, -1), ("bf16", 128, 64, 65, 1),
                                             ("f32", 64, 64, 300, 2)])
def test_forward_and_backward(dev, dtype, Dk, Dv, T, cp):
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_bwd, gdn_chunk_fwd
    x = gdn_inputs.generate(B=2, T=T, H=2, Dk=Dk, Dv=Dv, dtype=dtype, seed=600 + T + Dk, h0_std=0.3,
                            grad=True, dhT=True)
    x, gs = make_raw(x, 7 + T)
    print(f"[prep] T={T} Dk={Dk} Dv={Dv} {dtype} cp={cp}", flush=True)
    t = to_torch(x, dev)
    kw = kw_torch(gs, dev)
    o, hT = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, h0=t["h0"], cp_mode=cp, **kw)
    grads = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], h0=t["h0"], dhT=t["dhT"],
                          cp_mode=cp, **kw)
    torch.cuda.synchronize()
    okw = dict(qk_norm=True, gate_act=True, gate_scale=gs)
    want_o, want_h = prep.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, **okw)
    want = prep.bwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.do, x.h0, x.dhT, **okw)
    errs = dict(o=relerr(to_np(o), want_o), hT=relerr(to_np(hT), want_h))
    errs.update({n: relerr(to_np(a), want[n]) for n, a in zip(NAMES, grads)})
    print("    " + "  ".join(f"{k} {e:.3e}" for k, e in errs.items()), flush=True)
    bad = {k: e for k, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, bad


def test_saved_states_with_preprocessing(dev):
    """The forward's saved states and chunk matrices T feed the pre-processing
    backward like the recomputation does."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_bwd, gdn_chunk_fwd
    x = gdn_inputs.generate(B=1, T=333, H=2, Dk=128, Dv=128, dtype="bf16", seed=611, grad=True)
    x, gs = make_raw(x, 12)
    print("[prep] saved states", flush=True)
    t = to_torch(x, dev)
    kw = kw_torch(gs, dev)
    _, _, states, chunk_t = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, cp_mode=2,
                                          save_states=True, save_t=True, **kw)
    g1 = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], cp_mode=2, need_dh0=False, **kw)
    g2 = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], cp_mode=2, need_dh0=False,
                       states=states, **kw)
    g3 = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], cp_mode=2, need_dh0=False,
                       states=states, chunk_t=chunk_t, **kw)
    g4 = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], cp_mode=2, need_dh0=False,
                       chunk_t=chunk_t, **kw)
    torch.cuda.synchronize()
    for other in (g2, g3, g4):
        for n, a, b in zip(NAMES[:5], g1, other):
            assert relerr(to_np(b), to_np(a)) <= 1e-6, n


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode(dev, dtype):
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_decode_step
    x = gdn_inputs.generate(B=6, T=1, H=3, Dk=128, Dv=64, dtype=dtype, seed=620, h0_std=0.5)
    x, gs = make_raw(x, 13)
    print(f"[prep] decode {dtype}", flush=True)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tt = lambda a, d=dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)
    st = tt(x.h0, torch.float32)
    o = gdn_decode_step(tt(x.q[:, 0]), tt(x.k[:, 0]), tt(x.v[:, 0]), tt(x.g[:, 0], torch.float32), tt(x.beta[:, 0]),
                        x.scale, st, **kw_torch(gs, dev))
    torch.cuda.synchronize()
    want_o, want_h = prep.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, qk_norm=True, gate_act=True, gate_scale=gs)
    assert relerr(to_np(o), want_o[:, 0]) <= TOL[dtype]
    assert relerr(st.cpu().numpy(), want_h) <= TOL[dtype]
