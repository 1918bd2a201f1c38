"""Degenerate gates on the GPU, forward and backward against the fp64 oracle:
beta = 0 (nothing is written: the state only decays), g = 0 with beta = 0 (the
state is constant, so h_T equals h0 exactly), decay so strong that exp(cumsum g)
underflows inside a chunk, beta = 1 with unit keys (each write replaces the
state's component along k), and beta = 2.5 (writes that expand the state
along k, so the norm bound that sizes the lead-in has a positive term)."""
import numpy as np
import pytest

import gdn_inputs
from tests.helpers import relerr
from tests.test_gpu_backward import check_bwd
from tests.test_gpu_forward import check_fwd, run_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def base(dtype, seed, Dk=64, Dv=64, T=300):
    return gdn_inputs.generate(B=1, T=T, H=2, Dk=Dk, Dv=Dv, dtype=dtype, seed=seed, h0_std=0.5, grad=True,
                               dhT=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("cp", [-1, 1])
def test_no_write(dev, dtype, cp):
    """beta = 0: o_t = scale exp(cumsum g) h0^T q_t, h_T = exp(sum g) h0."""
    x = base(dtype, 801)
    x.beta = np.zeros_like(x.beta)
    check_fwd(x, dev, cp, "beta=0")
    check_bwd(x, dev, cp, "beta=0")


@pytest.mark.parametrize("cp", [-1, 1])
def test_constant_state(dev, cp):
    """g = 0 and beta = 0: h_T is h0 bit for bit, o_t = scale h0^T q_t."""
    x = base("f32", 802)
    x.beta = np.zeros_like(x.beta)
    x.g = np.zeros_like(x.g)
    o, hT = check_fwd(x, dev, cp, "g=0 beta=0")
    assert np.array_equal(hT, x.h0)
    check_bwd(x, dev, cp, "g=0 beta=0")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decay_underflow(dev, dtype):
    """g = -30 per token: exp of the in-chunk cumsum underflows to zero within
    a few tokens; only differences of cumsums may enter the products.  dg is
    then about 1e-13 of the terms it is formed from (T = 300 ends in a partial
    chunk, where the terms that cancel exactly are kept apart), and its largest
    entry comes from a single row term u_r . (dS' k_r) whose sum is about a
    hundredth of its parts: with U and the chunk-end gradient dS' rounded to
    bf16 that entry misses the bound (2.5e-2), so the kernels carry both to
    about 16 bits there.  Every tensor is held to the usual bound."""
    from oracle import ref
    from tests.test_gpu_backward import NAMES, run_bwd
    from tests.helpers import TOL
    x = base(dtype, 803)
    x.g = np.full_like(x.g, -30.0)
    want = ref.bwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.do, x.h0, x.dhT, x.cu_seqlens)
    for cp in (-1, 2):
        o, _ = check_fwd(x, dev, cp, "g=-30")
        assert np.isfinite(o).all()
        got = run_bwd(x, dev, cp)
        errs = {k: relerr(got[k], want[k]) for k in NAMES}
        print("    " + "  ".join(f"{k} {e:.3e}" for k, e in errs.items()), flush=True)
        bad = {k: e for k, e in errs.items() if not e <= TOL[dtype]}
        assert not bad, (cp, bad)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_full_replacement(dev, dtype):
    """beta = 1 with unit keys: I - k k^T is a projection (norm bound 1)."""
    x = base(dtype, 804, Dk=64, Dv=128 if dtype == "bf16" else 64)
    x.beta = np.ones_like(x.beta)
    for cp in (-1, 1):
        check_fwd(x, dev, cp, "beta=1")
        check_bwd(x, dev, cp, "beta=1")


def test_split_matches_unsplit_without_decay(dev):
    """g = 0 everywhere (no decay bound): every segment's lead-in reaches its
    sequence start, and the split run equals the unsplit one to fp32 rounding."""
    x = base("f32", 805, T=700)
    x.g = np.zeros_like(x.g)
    o_ref, h_ref = run_fwd(x, dev, -1)
    o, hT = run_fwd(x, dev, 1)
    assert relerr(o, o_ref) < 1e-5 and relerr(hT, h_ref) < 1e-5


def test_expanding_writes(dev):
    """beta = 2.5 with unit keys: ||I - beta k k^T|| = 1.5, so each chunk's
    log-bound carries 64 log 1.5 besides its decay (g = -0.485 per token leaves
    about -5 per chunk).  A lead-in sized without that term would stop four
    times too early; split and unsplit runs must still agree to fp32 rounding,
    forward and backward, and both match the oracle."""
    from tests.test_gpu_backward import NAMES, run_bwd
    rng = np.random.default_rng(806)
    x = base("f32", 806, T=640)
    x.beta = np.full_like(x.beta, 2.5)
    x.g = (-0.485 + 0.02 * rng.standard_normal(x.g.shape)).astype(np.float32)
    o_ref, h_ref = run_fwd(x, dev, -1)
    g_ref = run_bwd(x, dev, -1)
    for cp in (1, 3):
        o, hT = check_fwd(x, dev, cp, "beta=2.5")
        assert relerr(o, o_ref) < 1e-5 and relerr(hT, h_ref) < 1e-5, cp
        got, _ = check_bwd(x, dev, cp, "beta=2.5")
        for k in NAMES:
            assert relerr(got[k], g_ref[k]) < 1e-5, (cp, k)
