"""Forward parity on the GPU: HIP path through the C ABI vs the fp64 oracle,
element by element, on the same seeded inputs."""
import sys

import numpy as np
import pytest

import gdn_inputs
from oracle import ref
from tests.helpers import TOL, relerr, to_np, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_fwd(x, dev, cp_mode=0, final=True):
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    import torch
    t = to_torch(x, dev)
    host = None if x.cu_seqlens is None else x.cu_seqlens.astype(np.int32)
    o, hT = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, h0=t["h0"],
                          cu_seqlens=t["cu"], cu_seqlens_host=host, output_final_state=final,
                          cp_mode=cp_mode)
    torch.cuda.synchronize()
    return to_np(o), to_np(hT)


def check_fwd(x, dev, cp_mode=0, label=""):
    print(f"[fwd] {label} T={x.q.shape[1]} H={x.q.shape[2]} Dk={x.q.shape[3]} Dv={x.v.shape[3]} "
          f"{x.dtype} cp={cp_mode}", flush=True)
    sys.stdout.flush()
    o, hT = run_fwd(x, dev, cp_mode)
    ro, rhT = ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, x.h0, x.cu_seqlens)
    eo, eh = relerr(o, ro), relerr(hT, rhT)
    print(f"    o {eo:.3e}  hT {eh:.3e}", flush=True)
    assert eo <= TOL[x.dtype] and eh <= TOL[x.dtype], (eo, eh)
    return o, hT


# ------------------------------------------------------------------ small cases, many tiles + ragged tails
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 333])
@pytest.mark.parametrize("cp_mode", [-1, 1, 2])
def test_ragged_lengths_bf16(dev, T, cp_mode):
    x = gdn_inputs.generate(B=2, T=T, H=3, Dk=128, Dv=128, dtype="bf16", seed=100 + T, h0_std=0.5)
    check_fwd(x, dev, cp_mode, "ragged")


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (64, 128), (128, 64)])
def test_head_sizes_bf16(dev, Dk, Dv):
    x = gdn_inputs.generate(B=1, T=300, H=2, Dk=Dk, Dv=Dv, dtype="bf16", seed=7 + Dk + Dv, h0_std=0.1)
    for cp in (-1, 2):
        check_fwd(x, dev, cp, "heads")


@pytest.mark.parametrize("T,cp", [(256, -1), (256, 1), (130, 0), (700, 3)])
def test_fp32_path(dev, T, cp):
    x = gdn_inputs.generate(B=1, T=T, H=2, Dk=64, Dv=64, dtype="f32", seed=11 + T, h0_std=0.3)
    check_fwd(x, dev, cp, "f32")


def test_varlen_with_empty_and_tiny_sequences(dev):
    rng = np.random.default_rng(5)
    lens = [0, 1, 64, 130, 0, 77, 500, 3]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    y = gdn_inputs.generate(B=1, T=int(cu[-1]), H=2, Dk=128, Dv=128, dtype="bf16", seed=10)
    y.cu_seqlens = cu
    y.h0 = (0.3 * rng.standard_normal((len(lens), 2, 128, 128))).astype(np.float32)
    for cp in (-1, 1, 0):
        check_fwd(y, dev, cp, "varlen-edge")


@pytest.mark.parametrize("nseq", [64, 65, 300])
def test_many_sequences(dev, nseq):
    """Batches around and above 64 sequences (the plan's one-wave and block
    scans), with empty sequences among them."""
    rng = np.random.default_rng(nseq)
    lens = rng.integers(0, 90, size=nseq)
    lens[::7] = 0
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    y = gdn_inputs.generate(B=1, T=int(cu[-1]), H=1, Dk=64, Dv=64, dtype="bf16", seed=11)
    y.cu_seqlens = cu
    y.h0 = (0.3 * rng.standard_normal((nseq, 1, 64, 64))).astype(np.float32)
    for cp in (-1, 1):
        check_fwd(y, dev, cp, f"{nseq} sequences")


def test_segment_split_is_exact(dev):
    """With fp32 arithmetic throughout, forced segment splits agree with the
    unsplit run to fp32 rounding: the lead-in drops nothing."""
    x = gdn_inputs.generate(B=1, T=1000, H=2, Dk=64, Dv=64, dtype="f32", seed=3, h0_std=0.2)
    o_ref, h_ref = run_fwd(x, dev, -1)
    for cp in (1, 2, 5):
        o, hT = run_fwd(x, dev, cp)
        assert relerr(o, o_ref) < 1e-5 and relerr(hT, h_ref) < 1e-5, cp
    # bf16 inputs: split and unsplit both sit well inside the oracle tolerance
    y = gdn_inputs.generate(B=1, T=1000, H=2, Dk=128, Dv=128, dtype="bf16", seed=3, h0_std=0.2)
    for cp in (-1, 1, 5):
        check_fwd(y, dev, cp, "split-bf16")


def mixed_decay(x, seed):
    """Scale g chunk by chunk (factors 0.01 .. 6), so that the chunks' log-bounds
    range from about -0.05 to -30 and a segment's lead-in can be one chunk, a
    few chunks, or reach back to the sequence start."""
    rng = np.random.default_rng(seed)
    T = x.g.shape[1]
    f = rng.choice([0.01, 0.3, 1.0, 6.0], size=(T + 63) // 64)
    x.g = (x.g * np.repeat(f, 64)[:T][None, :, None]).astype(np.float32)
    return x


def test_lead_in_of_varying_length(dev):
    """Segments of one chunk whose lead-ins differ in length (mixed decay per
    chunk), fp32: equal to the oracle and to the unsplit run."""
    x = mixed_decay(gdn_inputs.generate(B=1, T=1200, H=2, Dk=64, Dv=64, dtype="f32", seed=21, h0_std=0.3), 5)
    o_ref, h_ref = run_fwd(x, dev, -1)
    for cp in (1, 3):
        o, hT = check_fwd(x, dev, cp, "mixed decay")
        assert relerr(o, o_ref) < 1e-5 and relerr(hT, h_ref) < 1e-5, cp


def test_slow_decay_falls_back_to_serial(dev):
    """Gates near zero do not decay across a segment: a segment's lead-in
    reaches back to the sequence start (from h0) -- results stay exact."""
    x = gdn_inputs.generate(B=1, T=640, H=2, Dk=128, Dv=128, dtype="bf16", seed=4, h0_std=0.2)
    x.g = (x.g * 1e-3).astype(np.float32)
    for cp in (1, 3):
        check_fwd(x, dev, cp, "no-decay")


def test_no_final_state(dev):
    x = gdn_inputs.generate(B=1, T=100, H=1, Dk=64, Dv=64, dtype="bf16", seed=1)
    o, hT = run_fwd(x, dev, 0, final=False)
    assert hT is None
    ro, _ = ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale)
    assert relerr(o, ro) <= TOL["bf16"]


def test_deterministic(dev):
    x = gdn_inputs.generate(B=1, T=777, H=2, Dk=128, Dv=128, dtype="bf16", seed=12, h0_std=0.1)
    a = run_fwd(x, dev, 2)
    b = run_fwd(x, dev, 2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ the measured workloads
@pytest.mark.parametrize("name", ["tiny_f32", "single_bf16", "long_fewhead", "varlen", "metric_32k"])
def test_config_forward(dev, name):
    x = gdn_inputs.config(name, grad=False)
    check_fwd(x, dev, 0, name)


@pytest.mark.parametrize("dtype,Dk,Dv,cp", [("bf16", 128, 128, 0), ("bf16", 64, 128, 2), ("bf16", 128, 64, -1),
                                           ("f32", 64, 64, 3)])
def test_saved_states_are_chunk_start_states(dev, dtype, Dk, Dv, cp):
    """Every saved state equals the oracle's state after the first 64 c tokens of
    its sequence (the initial state for c = 0), read back through the documented
    block layout, and every saved U (after the states) the oracle's chunk U."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    from tests.helpers import unblock_states
    lens = [130, 0, 64, 257, 5]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    x = gdn_inputs.generate(B=1, T=int(cu[-1]), H=2, Dk=Dk, Dv=Dv, dtype=dtype, seed=41 + Dk + Dv)
    x.cu_seqlens = cu
    x.h0 = (0.3 * np.random.default_rng(4).standard_normal((len(lens), 2, Dk, Dv))).astype(np.float32)
    print(f"[fwd] saved states {dtype} Dk={Dk} Dv={Dv} cp={cp}", flush=True)
    t = to_torch(x, dev)
    _, _, states = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, h0=t["h0"],
                                 cu_seqlens=t["cu"], cu_seqlens_host=cu, cp_mode=cp, save_states=True)
    torch.cuda.synchronize()
    C = sum((n + 63) // 64 for n in lens)
    got = unblock_states(to_np(states), C, 2, Dk, Dv)
    c = 0
    for n, ln in enumerate(lens):
        s0 = int(cu[n])
        for j in range((ln + 63) // 64):
            sl = slice(s0, s0 + 64 * j)
            want = x.h0[n] if j == 0 else ref.fwd(x.q[:, sl], x.k[:, sl], x.v[:, sl], x.g[:, sl], x.beta[:, sl],
                                                  x.scale, x.h0[n:n + 1])[1][0]
            err = relerr(got[c], want)
            assert err <= TOL[dtype], (n, j, err)
            c += 1
    assert c == C
    from oracle import chunked
    want_u = chunked.chunk_u(x.k, x.v, x.g, x.beta, x.h0, cu)
    flat = to_np(states).astype(np.float64)
    # [C, H, Dv/16, 64, 16] column blocks -> [C, H, 64, Dv]
    got_u = flat[C * 2 * Dk * Dv:C * 2 * Dk * Dv + want_u.size].reshape(C, 2, Dv // 16, 64, 16)
    got_u = got_u.transpose(0, 1, 3, 2, 4).reshape(want_u.shape)
    err = relerr(got_u, want_u)
    print(f"    U {err:.3e}", flush=True)
    assert err <= TOL[dtype]
    if dtype == "bf16":
        # then U's rounding residual, laid out as U: below half a bf16 step of U
        # itself, and U + residual still the oracle's U
        off = C * 2 * (Dk * Dv + 64 * Dv)
        lo = flat[off:off + want_u.size].reshape(C, 2, Dv // 16, 64, 16).transpose(0, 1, 3, 2, 4).reshape(want_u.shape)
        assert np.all(np.abs(lo) <= np.abs(got_u) * 2.0 ** -8 + 1e-30)
        err2 = relerr(got_u + lo, want_u)
        print(f"    U + residual {err2:.3e}", flush=True)
        assert err2 <= TOL[dtype]


@pytest.mark.parametrize("dtype,Dk,Dv,cp", [("bf16", 128, 128, 0), ("bf16", 64, 128, 3), ("f32", 64, 64, -1)])
def test_saved_t_matches_oracle(dev, dtype, Dk, Dv, cp):
    """Every saved chunk matrix T equals the oracle's (the chunked form's T,
    completed with the identity past a sequence end), entry by entry."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    from oracle import chunked
    lens = [130, 0, 64, 257, 5]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    x = gdn_inputs.generate(B=1, T=int(cu[-1]), H=2, Dk=Dk, Dv=Dv, dtype=dtype, seed=52 + Dk + Dv)
    x.cu_seqlens = cu
    print(f"[fwd] saved T {dtype} Dk={Dk} Dv={Dv} cp={cp}", flush=True)
    t = to_torch(x, dev)
    res = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, cu_seqlens=t["cu"],
                        cu_seqlens_host=cu, cp_mode=cp, save_t=True)
    torch.cuda.synchronize()
    want = chunked.chunk_t(x.k, x.g, x.beta, cu)
    raw = res[2][:want.size]
    if dtype == "bf16":
        # each 64 x 64 entry holds T's bf16 value plane, then its residual plane
        planes = raw.view(torch.bfloat16).reshape(-1, 2, 64 * 64).cpu().double().numpy()
        lo_rel = np.abs(planes[:, 1]).max() / np.abs(planes[:, 0]).max()
        assert lo_rel <= 2.0 ** -8, lo_rel  # the residual is below the value's rounding step
        got = (planes[:, 0] + planes[:, 1]).reshape(want.shape)
    else:
        got = raw.cpu().numpy().astype(np.float64).reshape(want.shape)
    err = relerr(got, want)
    print(f"    T {err:.3e}", flush=True)
    # T is formed and solved in fp32 from the exact (dtype-rounded) inputs in
    # both dtypes (for bf16 inputs stored as value + residual, about 16 bits),
    # so it is held to the fp32 bound
    assert err <= TOL["f32"]


@pytest.mark.parametrize("cp", [-1, 2])
def test_saved_scalar_record(dev, cp):
    """The scalar record saved after the chunk matrices (gdn_chunk_t_bytes):
    decay cumsum G and its exponentials, beta, beta exp(G), the log-bound Lambda
    and exp(G_63) of every chunk, against their definitions in float64."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    lens = [130, 0, 64, 257, 5]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    H = 2
    x = gdn_inputs.generate(B=1, T=int(cu[-1]), H=H, Dk=128, Dv=128, dtype="bf16", seed=57)
    x.cu_seqlens = cu
    print(f"[fwd] saved scalar record cp={cp}", flush=True)
    t = to_torch(x, dev)
    res = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, cu_seqlens=t["cu"],
                        cu_seqlens_host=cu, cp_mode=cp, save_t=True)
    torch.cuda.synchronize()
    flat = res[2].cpu().numpy().astype(np.float64)
    nch = sum((n + 63) // 64 for n in lens)
    rec = flat[nch * H * 4096:nch * H * (4096 + 324)].reshape(nch, H, 324)
    g, beta, k = (np.asarray(a, dtype=np.float64) for a in (x.g[0], x.beta[0], x.k[0]))
    want = np.zeros_like(rec)
    c = 0
    for n, L in enumerate(lens):
        for j in range((L + 63) // 64):
            rows = min(64, L - 64 * j)
            s0 = cu[n] + 64 * j
            for h in range(H):
                gg = np.zeros(64); bb = np.zeros(64); kk2 = np.zeros(64)
                gg[:rows] = g[s0:s0 + rows, h]
                bb[:rows] = beta[s0:s0 + rows, h]
                kk2[:rows] = np.sum(k[s0:s0 + rows, h] ** 2, axis=-1)
                G = np.cumsum(gg)
                want[c, h, 0:64] = G
                want[c, h, 64:128] = np.exp(G)
                want[c, h, 128:192] = np.exp(G[63] - G)
                want[c, h, 192:256] = bb
                want[c, h, 256:320] = bb * np.exp(G)
                want[c, h, 320] = np.sum(gg + np.log(np.maximum(1.0, np.abs(1.0 - bb * kk2))))
                want[c, h, 321] = np.exp(G[63])
            c += 1
    for lo, hi, name in ((0, 64, "G"), (64, 128, "exp G"), (128, 192, "exp(G_C - G)"), (192, 256, "beta"),
                         (256, 320, "beta exp G"), (320, 321, "Lambda"), (321, 324, "exp G_C, 0, 0")):
        err = relerr(rec[..., lo:hi], want[..., lo:hi])
        print(f"    {name} {err:.3e}", flush=True)
        assert err <= 1e-5, name


@pytest.mark.parametrize("dev_lens", [[64, 236], [100, 150]])
def test_device_cu_seqlens_mismatch_writes_nothing(dev, dev_lens):
    """The host copy of cu_seqlens sizes the work; a device copy that gives
    other chunk totals (64 + 236 tokens: 5 chunks, not 2 + 4) or does not end
    at T (100 + 150 of 300 tokens) makes the kernels write nothing."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    host = np.array([0, 100, 300], dtype=np.int32)
    devcu = np.concatenate([[0], np.cumsum(dev_lens)]).astype(np.int32)
    x = gdn_inputs.generate(B=1, T=300, H=2, Dk=64, Dv=64, dtype="bf16", seed=61)
    print(f"[fwd] cu_seqlens mismatch device {devcu.tolist()} host {host.tolist()}", flush=True)
    t = to_torch(x, dev)
    o = torch.full((1, 300, 2, 64), 7.0, dtype=torch.bfloat16, device=dev)
    hT = torch.full((2, 2, 64, 64), 7.0, dtype=torch.float32, device=dev)
    gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale, cu_seqlens=torch.from_numpy(devcu).to(dev),
                  cu_seqlens_host=host, cp_mode=1, o=o, hT=hT)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((hT == 7.0).all())


def test_device_cu_seqlens_same_totals_follows_device(dev):
    """A device copy with the host copy's totals (200 + 100 tokens: 4 + 2
    chunks, as 100 + 200) is what the kernels follow."""
    import torch
    from gated_deltanet_chunked_delta_amd import gdn_chunk_fwd
    host = np.array([0, 100, 300], dtype=np.int32)
    devcu = np.array([0, 200, 300], dtype=np.int32)
    x = gdn_inputs.generate(B=1, T=300, H=2, Dk=64, Dv=64, dtype="bf16", seed=62)
    print("[fwd] cu_seqlens same totals", flush=True)
    t = to_torch(x, dev)
    o, hT = gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], x.scale,
                          cu_seqlens=torch.from_numpy(devcu).to(dev), cu_seqlens_host=host, cp_mode=1)
    torch.cuda.synchronize()
    ro, rhT = ref.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, None, devcu)
    assert relerr(to_np(o), ro) <= TOL["bf16"] and relerr(to_np(hT), rhT) <= TOL["bf16"]
