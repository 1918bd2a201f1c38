"""The allocation-free forward (gdn_chunk_fwd_noalloc) on the GPU: the same
kernels as gdn_chunk_fwd with the library's own scratch in place of the
caller's workspace, so its outputs must equal gdn_chunk_fwd's bit for bit.
Two calls in a row, the second smaller than the first (the scratch keeps the
first call's contents), with and without the caller keeping T."""
import numpy as np
import pytest

import gdn_inputs
from tests.helpers import to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run(x, dev, cp, save_t, noalloc):
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    t = to_torch(x, dev)
    res = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, h0=t["h0"], cu_seqlens=t["cu"],
                        cu_seqlens_host=x.cu_seqlens, cp_mode=cp, save_t=save_t, noalloc=noalloc)
    torch.cuda.synchronize()
    return [r.float().cpu().numpy() for r in res]


@pytest.mark.parametrize("save_t", [False, True])
def test_noalloc_matches_workspace_call(dev, save_t):
    # first call: 8 sequences of mixed length (60 chunk-heads x 16 heads), then a
    # smaller one (1 sequence, 3 chunks, 2 heads)
    rng = np.random.default_rng(71)
    lens = rng.integers(1, 400, size=8)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    big = gdn_inputs.generate(B=1, T=int(cu[-1]), H=16, Dk=128, Dv=128, dtype="bf16", seed=72, h0_std=0.02)
    big.cu_seqlens = cu
    big.h0 = (0.02 * rng.standard_normal((len(lens), 16, 128, 128))).astype(np.float32)
    small = gdn_inputs.generate(B=1, T=150, H=2, Dk=64, Dv=64, dtype="bf16", seed=73, h0_std=0.02)
    for name, x, cp in (("8 sequences, H=16, d=128", big, 0), ("T=150, H=2, d=64", small, 1)):
        print(f"[noalloc] {name} save_t={save_t}", flush=True)
        want = run(x, dev, cp, save_t, noalloc=False)
        got = run(x, dev, cp, save_t, noalloc=True)
        assert len(got) == len(want)
        for g_, w_ in zip(got, want):
            assert np.array_equal(g_, w_), name
