"""Decode-step parity on the GPU: gdn_decode_step through the C ABI against the
fp64 oracle's token recurrence (one token with h0 = the state), element by
element on the same seeded inputs; continuation of a chunked prefill; state
slots and padding entries."""
import numpy as np
import pytest

import gdn_inputs
from oracle import ref
from tests.helpers import TOL, relerr, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def tens(a, dev, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dtype).contiguous()


def one_step(x, dev, state_np):
    """Run one decode step for the T = 1 inputs of x; returns (o, new state) as numpy."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_decode_step
    dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    q, k, v = (tens(a[:, 0], dev, dt) for a in (x.q, x.k, x.v))
    beta = tens(x.beta[:, 0], dev, dt)
    g = tens(x.g[:, 0], dev, torch.float32)
    st = tens(state_np, dev, torch.float32)
    o = gdn_decode_step(q, k, v, g, beta, x.scale, st)
    torch.cuda.synchronize()
    return to_np(o), st.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_one_step_matches_recurrence(dev, dtype, Dk, Dv):
    x = gdn_inputs.generate(B=5, T=1, H=3, Dk=Dk, Dv=Dv, dtype=dtype, seed=500 + Dk + Dv, h0_std=0.5)
    print(f"[decode] N=5 H=3 Dk={Dk} Dv={Dv} {dtype}", flush=True)
    o, st = one_step(x, dev, x.h0)
    want_o, want_h = ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0)
    eo, eh = relerr(o, want_o[:, 0]), relerr(st, want_h)
    print(f"    o {eo:.3e}  state {eh:.3e}", flush=True)
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


def test_prefill_then_decode(dev):
    """gdn_chunk_fwd over T tokens (hT), then the next tokens one decode step at a
    time, equals the recurrence over all tokens."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd, gdn_decode_step
    T0, extra = 200, 6
    x = gdn_inputs.generate(B=2, T=T0 + extra, H=2, Dk=128, Dv=128, dtype="bf16", seed=77, h0_std=0.3)
    print(f"[decode] prefill {T0} + {extra} steps", flush=True)
    bf = torch.bfloat16
    sl = lambda a, lo, hi: np.ascontiguousarray(a[:, lo:hi])
    _, hT = gdn_chunk_fwd(tens(sl(x.q, 0, T0), dev, bf), tens(sl(x.k, 0, T0), dev, bf), tens(sl(x.v, 0, T0), dev, bf),
                          tens(sl(x.g, 0, T0), dev, torch.float32), tens(sl(x.beta, 0, T0), dev, bf), x.scale,
                          h0=tens(x.h0, dev, torch.float32))
    outs = []
    for t in range(T0, T0 + extra):
        outs.append(gdn_decode_step(tens(x.q[:, t], dev, bf), tens(x.k[:, t], dev, bf), tens(x.v[:, t], dev, bf),
                                    tens(x.g[:, t], dev, torch.float32), tens(x.beta[:, t], dev, bf), x.scale, hT))
    torch.cuda.synchronize()
    want_o, want_h = ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0)
    o = np.stack([to_np(a) for a in outs], axis=1)
    eo, eh = relerr(o, want_o[:, T0:]), relerr(hT.cpu().numpy(), want_h)
    print(f"    o {eo:.3e}  state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


def test_state_slots_and_padding(dev):
    """Sequence n updates slot state_idx[n]; out-of-range indices are padding (no
    write of o, no state change); other slots keep their contents bit for bit."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_decode_step
    N, S, H = 6, 9, 2
    x = gdn_inputs.generate(B=N, T=1, H=H, Dk=64, Dv=128, dtype="bf16", seed=88)
    rng = np.random.default_rng(3)
    states = (0.4 * rng.standard_normal((S, H, 64, 128))).astype(np.float32)
    idx = np.array([7, -1, 2, 0, 9, 4], dtype=np.int32)     # two padding entries
    print("[decode] slots", idx.tolist(), flush=True)
    bf = torch.bfloat16
    st = tens(states, dev, torch.float32)
    o = torch.full((N, H, 128), 7.0, dtype=bf, device=dev)
    gdn_decode_step(tens(x.q[:, 0], dev, bf), tens(x.k[:, 0], dev, bf), tens(x.v[:, 0], dev, bf),
                    tens(x.g[:, 0], dev, torch.float32), tens(x.beta[:, 0], dev, bf), x.scale, st,
                    state_idx=torch.from_numpy(idx).to(dev), o=o)
    torch.cuda.synchronize()
    got_st, got_o = st.cpu().numpy(), to_np(o)
    for n, s in enumerate(idx):
        if 0 <= s < S:
            sel = slice(n, n + 1)
            want_o, want_h = ref.fwd(x.q[sel], x.k[sel], x.v[sel], x.g[sel], x.beta[sel], x.scale, states[s:s + 1])
            assert relerr(got_o[n], want_o[0, 0]) <= TOL["bf16"]
            assert relerr(got_st[s], want_h[0]) <= TOL["bf16"]
        else:
            assert np.all(got_o[n] == 7.0)
    untouched = sorted(set(range(S)) - {int(s) for s in idx if 0 <= s < S})
    assert np.array_equal(got_st[untouched], states[untouched])


def test_full_size_batch(dev):
    """The measured decode workload (64 sequences x 16 heads, d = 128, bf16): every
    output, and the states of a sample of (sequence, head) pairs."""
    x = gdn_inputs.generate(B=64, T=1, H=16, Dk=128, Dv=128, dtype="bf16", seed=20260099, h0_std=0.1)
    print("[decode] N=64 H=16 d=128 bf16", flush=True)
    o, st = one_step(x, dev, x.h0)
    want_o, want_h = ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0)
    assert relerr(o, want_o[:, 0]) <= TOL["bf16"]
    assert relerr(st, want_h) <= TOL["bf16"]
