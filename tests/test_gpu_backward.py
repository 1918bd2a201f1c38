"""Backward parity on the GPU: all six gradients through the C ABI vs the fp64
oracle's reverse-mode derivative, element by element, on the same seeded inputs."""
import numpy as np
import pytest

import gdn_inputs
from oracle import ref
from tests.helpers import TOL, relerr, to_np, to_torch

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_bwd(x, dev, cp_mode=0):
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_bwd
    t = to_torch(x, dev)
    host = None if x.cu_seqlens is None else x.cu_seqlens.astype(np.int32)
    out = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], h0=t["h0"],
                        dhT=t["dhT"], cu_seqlens=t["cu"], cu_seqlens_host=host, cp_mode=cp_mode)
    torch.cuda.synchronize()
    return dict(zip(NAMES, (to_np(a) for a in out)))


def check_bwd(x, dev, cp_mode=0, label=""):
    print(f"[bwd] {label} B={x.q.shape[0]} T={x.q.shape[1]} H={x.q.shape[2]} Dk={x.q.shape[3]} "
          f"Dv={x.v.shape[3]} {x.dtype} cp={cp_mode}", flush=True)
    got = run_bwd(x, dev, cp_mode)
    want = ref.bwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.do, x.h0, x.dhT, x.cu_seqlens)
    errs = {k: relerr(got[k], want[k]) for k in NAMES}
    print("    " + "  ".join(f"{k} {e:.3e}" for k, e in errs.items()), flush=True)
    bad = {k: e for k, e in errs.items() if not e <= TOL[x.dtype]}
    assert not bad, bad
    return got, want


@pytest.mark.parametrize("T", [1, 64, 65, 200])
@pytest.mark.parametrize("cp_mode", [-1, 1, 2])
def test_ragged_bf16(dev, T, cp_mode):
    x = gdn_inputs.generate(B=2, T=T, H=2, Dk=128, Dv=128, dtype="bf16", seed=300 + T, h0_std=0.5,
                            grad=True, dhT=True)
    check_bwd(x, dev, cp_mode, "ragged")


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
def test_head_sizes_bf16(dev, Dk, Dv):
    x = gdn_inputs.generate(B=1, T=300, H=2, Dk=Dk, Dv=Dv, dtype="bf16", seed=31 + Dk + Dv, h0_std=0.1,
                            grad=True, dhT=True)
    for cp in (-1, 2):
        check_bwd(x, dev, cp, "heads")


@pytest.mark.parametrize("T,cp", [(256, -1), (256, 1), (190, 0), (700, 3)])
def test_fp32_path(dev, T, cp):
    x = gdn_inputs.generate(B=1, T=T, H=2, Dk=64, Dv=64, dtype="f32", seed=41 + T, h0_std=0.3,
                            grad=True, dhT=True)
    check_bwd(x, dev, cp, "f32")


def test_varlen_with_empty_and_tiny_sequences(dev):
    rng = np.random.default_rng(6)
    lens = [0, 1, 64, 130, 0, 77, 500, 3]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    x = gdn_inputs.generate(B=1, T=int(cu[-1]), H=2, Dk=128, Dv=128, dtype="bf16", seed=16, grad=True)
    x.cu_seqlens = cu
    x.h0 = (0.3 * rng.standard_normal((len(lens), 2, 128, 128))).astype(np.float32)
    x.dhT = rng.standard_normal((len(lens), 2, 128, 128)).astype(np.float32)
    for cp in (-1, 1, 0):
        check_bwd(x, dev, cp, "varlen-edge")


def test_lead_in_of_varying_length(dev):
    """Segments of one chunk whose lead-ins (after the segment, in the reverse
    chain) differ in length, fp32: equal to the oracle and to the unsplit run."""
    from tests.test_gpu_forward import mixed_decay
    x = mixed_decay(gdn_inputs.generate(B=1, T=1200, H=2, Dk=64, Dv=64, dtype="f32", seed=22, h0_std=0.3,
                                        grad=True, dhT=True), 6)
    base = run_bwd(x, dev, -1)
    for cp in (1, 3):
        got, _ = check_bwd(x, dev, cp, "mixed decay")
        for k in NAMES:
            assert relerr(got[k], base[k]) < 1e-5, (cp, k)


def test_slow_decay_falls_back_to_serial(dev):
    """Gates near zero: every lead-in reaches the sequence end (from dhT)."""
    x = gdn_inputs.generate(B=1, T=640, H=2, Dk=128, Dv=128, dtype="bf16", seed=17, h0_std=0.2,
                            grad=True, dhT=True)
    x.g = (x.g * 1e-3).astype(np.float32)
    for cp in (1, 3):
        check_bwd(x, dev, cp, "no-decay")


def test_segment_split_is_exact_fp32(dev):
    x = gdn_inputs.generate(B=1, T=1000, H=2, Dk=64, Dv=64, dtype="f32", seed=18, h0_std=0.2,
                            grad=True, dhT=True)
    base = run_bwd(x, dev, -1)
    for cp in (1, 2, 5):
        got = run_bwd(x, dev, cp)
        for k in NAMES:
            assert relerr(got[k], base[k]) < 1e-5, (cp, k)


def test_no_initial_state_gradient(dev):
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_bwd
    x = gdn_inputs.generate(B=1, T=100, H=2, Dk=64, Dv=64, dtype="bf16", seed=19, grad=True)
    t = to_torch(x, dev)
    out = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], need_dh0=False)
    torch.cuda.synchronize()
    assert out[5] is None
    want = ref.bwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.do)
    for name, got in zip(NAMES[:5], out[:5]):
        assert relerr(to_np(got), want[name]) <= TOL["bf16"], name


def test_euler_identities_on_gpu_output(dev):
    """sum do.o + <dhT, hT> = sum dv.v + <dh0, h0>  and  sum dq.q = sum do.o,
    both exact for the gated delta rule (o and hT are degree-1 homogeneous in
    (v, h0), and o is linear in q); checked on the GPU's own outputs."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    x = gdn_inputs.generate(B=2, T=777, H=4, Dk=128, Dv=128, dtype="bf16", seed=20, h0_std=0.2,
                            grad=True, dhT=True)
    t = to_torch(x, dev)
    o, hT = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, h0=t["h0"], cp_mode=2)
    torch.cuda.synchronize()
    gr = run_bwd(x, dev, 2)
    o, hT = to_np(o).astype(np.float64), to_np(hT).astype(np.float64)
    lhs = np.sum(x.do * o) + np.sum(x.dhT * hT)
    rhs = np.sum(gr["dv"] * x.v) + np.sum(gr["dh0"] * x.h0)
    assert abs(lhs - rhs) <= 2e-2 * (np.abs(x.do * o).sum() + np.abs(x.dhT * hT).sum())
    assert abs(np.sum(gr["dq"] * x.q) - np.sum(x.do * o)) <= 2e-2 * np.abs(x.do * o).sum()


# ------------------------------------------------------------------ the measured workloads
@pytest.mark.parametrize("name", ["train", "metric_32k"])
def test_config_backward(dev, name):
    x = gdn_inputs.config(name)
    check_bwd(x, dev, 0, name)


@pytest.mark.parametrize("cp_mode,save_s,save_t", [(-1, True, False), (2, True, False), (0, True, False),
                                                   (2, False, True), (0, True, True)])
def test_saved_states_match_replay(dev, cp_mode, save_s, save_t):
    """The backward fed with the forward's saved chunk states and / or chunk
    matrices T gives the same gradients as the backward that recomputes them
    (same kernels, same arithmetic order), and the forward's outputs do not
    change by saving them."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_bwd, gdn_chunk_fwd
    rng = np.random.default_rng(9)
    lens = [0, 70, 300, 1, 129]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    x = gdn_inputs.generate(B=1, T=int(cu[-1]), H=2, Dk=128, Dv=128, dtype="bf16", seed=91, grad=True)
    x.cu_seqlens = cu
    x.h0 = (0.3 * rng.standard_normal((len(lens), 2, 128, 128))).astype(np.float32)
    x.dhT = rng.standard_normal((len(lens), 2, 128, 128)).astype(np.float32)
    print(f"[bwd] saved states={save_s} T={save_t} varlen cp={cp_mode}", flush=True)
    t = to_torch(x, dev)
    kw = dict(h0=t["h0"], cu_seqlens=t["cu"], cu_seqlens_host=cu, cp_mode=cp_mode)
    o1, hT1 = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, **kw)
    res = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, save_states=save_s, save_t=save_t,
                        **kw)
    o2, hT2 = res[0], res[1]
    states = res[2] if save_s else None
    chunk_t = res[-1] if save_t else None
    g1 = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], dhT=t["dhT"], **kw)
    g2 = gdn_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, t["do"], dhT=t["dhT"],
                       states=states, chunk_t=chunk_t, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(hT1, hT2)
    for name, a, b in zip(NAMES, g1, g2):
        da, db = to_np(a), to_np(b)
        err = relerr(db, da)
        print(f"    {name} {err:.3e}", flush=True)
        assert err <= 1e-6, (name, err)
    want = ref.bwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.do, x.h0, x.dhT, x.cu_seqlens)
    for name, b in zip(NAMES, g2):
        assert relerr(to_np(b), want[name]) <= TOL[x.dtype], name
