"""Pins for the fp64 oracle: closed forms, special cases, invariants, finite
differences and a hand-worked example -- nothing here re-derives the oracle's
own loop.  All CPU-only."""
import json
import os

import numpy as np
import pytest

from oracle import chunked, ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, B=1, T=37, H=2, Dk=5, Dv=4, unit_k=True, h0=True, decay=0.3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -rng.random((B, T, H)) * decay
    beta = rng.random((B, T, H))
    hh = rng.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, hh


def relerr(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------- hand example
def test_golden_two_tokens_by_hand():
    d = json.load(open(os.path.join(GOLD, "two_token_by_hand.json")))
    arr = {key: np.array(val, dtype=np.float64) for key, val in d.items() if isinstance(val, list)}
    o, hT = ref.fwd(arr["q"], arr["k"], arr["v"], arr["g"], arr["beta"], d["scale"])
    np.testing.assert_allclose(o, arr["o"], atol=1e-14)
    np.testing.assert_allclose(hT, arr["hT"], atol=1e-14)
    gr = ref.bwd(arr["q"], arr["k"], arr["v"], arr["g"], arr["beta"], d["scale"], arr["do"])
    for name in ("dq", "dk", "dv", "dbeta", "dg", "dh0"):
        np.testing.assert_allclose(gr[name], arr[name], atol=1e-14, err_msg=name)


# ---------------------------------------------------------------- I1: one step
def test_single_token_closed_form():
    q, k, v, g, beta, h0 = rand_case(1, T=1, Dk=4, Dv=3)
    S0 = h0[0, 1].T  # dv x dk
    kk, vv, qq = k[0, 0, 1], v[0, 0, 1], q[0, 0, 1]
    a, b = np.exp(g[0, 0, 1]), beta[0, 0, 1]
    S1 = a * S0 @ (np.eye(4) - b * np.outer(kk, kk)) + b * np.outer(vv, kk)
    o, hT = ref.fwd(q, k, v, g, beta, 0.3, h0)
    np.testing.assert_allclose(o[0, 0, 1], 0.3 * S1 @ qq, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(hT[0, 1], S1.T, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- I2: beta = 0
def test_beta_zero_is_pure_decay():
    q, k, v, g, beta, h0 = rand_case(2, T=29)
    beta[:] = 0.0
    o, hT = ref.fwd(q, k, v, g, beta, 0.5, h0)
    gam = np.cumsum(g, axis=1)  # [B,T,H]
    for h in range(2):
        S0 = h0[0, h].T
        exp_o = 0.5 * np.exp(gam[0, :, h])[:, None] * (q[0, :, h] @ S0.T)
        np.testing.assert_allclose(o[0, :, h], exp_o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(hT[0, h], np.exp(gam[0, -1, h]) * h0[0, h], rtol=1e-12)
    o0, hT0 = ref.fwd(q, k, v, g, beta, 0.5, None)
    assert np.all(o0 == 0) and np.all(hT0 == 0)


# ---------------------------------------------------------------- I3: GLA limit
def test_small_beta_limit_is_gated_linear_attention():
    q, k, v, g, beta, h0 = rand_case(3, T=23, unit_k=False)
    eps = 2.0 ** -30
    beta[:] = eps
    vhat = v.copy()
    o, _ = ref.fwd(q, k, vhat / eps, g, beta, 0.7, h0)
    gam = np.cumsum(g, axis=1)
    T = q.shape[1]
    for h in range(2):
        G = gam[0, :, h]
        Dm = np.exp(G[:, None] - G[None, :]) * np.tril(np.ones((T, T)))
        att = (q[0, :, h] @ k[0, :, h].T) * Dm
        expect = 0.7 * (att @ vhat[0, :, h] + np.exp(G)[:, None] * (q[0, :, h] @ h0[0, h]))
        assert relerr(o[0, :, h], expect) < 1e-6


# ---------------------------------------------------------------- I4: g = 0, beta = 0
def test_constant_state():
    q, k, v, g, beta, h0 = rand_case(4, T=17)
    g[:] = 0.0
    beta[:] = 0.0
    o, hT = ref.fwd(q, k, v, g, beta, 1.1, h0)
    np.testing.assert_array_equal(hT, h0)
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h], 1.1 * q[0, :, h] @ h0[0, h], rtol=1e-13)


# ---------------------------------------------------------------- I5: delta-rule retrieval
def test_unit_beta_retrieves_value():
    q, k, v, g, beta, h0 = rand_case(5, T=19, Dk=6, Dv=3)
    beta[:] = 1.0
    o, _ = ref.fwd(k, k, v, g, beta, 1.0, h0)  # q = k reads S_t k_t
    np.testing.assert_allclose(o, v, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- I6: basis keys
def test_basis_keys_column_recurrence():
    rng = np.random.default_rng(6)
    T, Dk, Dv = 25, 4, 3
    idx = rng.integers(0, Dk, size=T)
    k = np.zeros((1, T, 1, Dk))
    k[0, np.arange(T), 0, idx] = 1.0
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    g = -rng.random((1, T, 1)) * 0.5
    beta = rng.random((1, T, 1)) * 2.0
    h0 = rng.standard_normal((1, 1, Dk, Dv))
    o, hT = ref.fwd(q, k, v, g, beta, 1.0, h0)
    cols = [h0[0, 0, j].copy() for j in range(Dk)]  # column j of S = row j of h
    for t in range(T):
        a, b, j = np.exp(g[0, t, 0]), beta[0, t, 0], idx[t]
        for c in range(Dk):
            cols[c] = a * cols[c] if c != j else a * (1 - b) * cols[c] + b * v[0, t, 0]
        expect = sum(cols[c] * q[0, t, 0, c] for c in range(Dk))
        np.testing.assert_allclose(o[0, t, 0], expect, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hT[0, 0], np.stack(cols), rtol=1e-12)


# ---------------------------------------------------------------- I7: chunked == sequential
@pytest.mark.parametrize("C", [1, 2, 8, 16, 64, 128])
def test_chunked_form_equals_recurrence(C):
    q, k, v, g, beta, h0 = rand_case(7, B=2, T=67, Dk=5, Dv=4)
    rng = np.random.default_rng(70)
    do = rng.standard_normal(v.shape)
    dhT = rng.standard_normal(h0.shape)
    o, hT = ref.fwd(q, k, v, g, beta, 0.6, h0)
    o2, hT2 = chunked.fwd(q, k, v, g, beta, 0.6, h0, C=C)
    assert relerr(o2, o) < 1e-12 and relerr(hT2, hT) < 1e-12
    a = ref.bwd(q, k, v, g, beta, 0.6, do, h0, dhT)
    b = chunked.bwd(q, k, v, g, beta, 0.6, do, h0, dhT, C=C)
    for name in a:
        assert relerr(b[name], a[name]) < 1e-12, name


# ---------------------------------------------------------------- I8: split call
def test_split_call_equals_single_call():
    q, k, v, g, beta, h0 = rand_case(8, T=150)
    rng = np.random.default_rng(80)
    do = rng.standard_normal(v.shape)
    tau = 71
    o, hT = ref.fwd(q, k, v, g, beta, 0.5, h0)
    sl = lambda x, a, b: x[:, a:b]
    oa, ha = ref.fwd(*(sl(x, 0, tau) for x in (q, k, v, g, beta)), 0.5, h0)
    ob, hb = ref.fwd(*(sl(x, tau, 150) for x in (q, k, v, g, beta)), 0.5, ha)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hb, hT, rtol=1e-12)
    full = ref.bwd(q, k, v, g, beta, 0.5, do, h0)
    second = ref.bwd(*(sl(x, tau, 150) for x in (q, k, v, g, beta)), 0.5, sl(do, tau, 150), ha)
    first = ref.bwd(*(sl(x, 0, tau) for x in (q, k, v, g, beta)), 0.5, sl(do, 0, tau), h0,
                    dhT=second["dh0"])
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        np.testing.assert_allclose(np.concatenate([first[name], second[name]], 1), full[name],
                                   rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(first["dh0"], full["dh0"], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- I9: varlen
def test_packed_varlen_equals_per_sequence():
    lens = [5, 64, 1, 70]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = rand_case(9, T=int(cu[-1]))
    rng = np.random.default_rng(90)
    h0 = rng.standard_normal((len(lens), 2, 5, 4))
    do = rng.standard_normal(v.shape)
    o, hT = ref.fwd(q, k, v, g, beta, 0.4, h0, cu_seqlens=cu)
    gr = ref.bwd(q, k, v, g, beta, 0.4, do, h0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sl = lambda x: x[:, a:b]
        on, hn = ref.fwd(*(sl(x) for x in (q, k, v, g, beta)), 0.4, h0[n:n + 1])
        np.testing.assert_allclose(o[:, a:b], on, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(hT[n], hn[0], rtol=1e-13)
        gn = ref.bwd(*(sl(x) for x in (q, k, v, g, beta)), 0.4, sl(do), h0[n:n + 1])
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_allclose(gr[name][:, a:b], gn[name], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gr["dh0"][n], gn["dh0"][0], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- I10: linearity in (v, h0)
def test_linear_in_values_and_initial_state():
    q, k, v, g, beta, h0 = rand_case(10, T=41)
    rng = np.random.default_rng(100)
    v2, h2 = rng.standard_normal(v.shape), rng.standard_normal(h0.shape)
    o1, t1 = ref.fwd(q, k, v, g, beta, 0.5, h0)
    o2, t2 = ref.fwd(q, k, v2, g, beta, 0.5, h2)
    o3, t3 = ref.fwd(q, k, 2.0 * v - 3.0 * v2, g, beta, 0.5, 2.0 * h0 - 3.0 * h2)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(t3, 2 * t1 - 3 * t2, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- I11: Euler identities
def test_euler_identities():
    q, k, v, g, beta, h0 = rand_case(11, B=2, T=45)
    rng = np.random.default_rng(110)
    do, dhT = rng.standard_normal(v.shape), rng.standard_normal(h0.shape)
    o, hT = ref.fwd(q, k, v, g, beta, 0.8, h0)
    gr = ref.bwd(q, k, v, g, beta, 0.8, do, h0, dhT)
    lhs = np.sum(do * o) + np.sum(dhT * hT)
    np.testing.assert_allclose(np.sum(gr["dv"] * v) + np.sum(gr["dh0"] * h0), lhs, rtol=1e-11)
    np.testing.assert_allclose(np.sum(gr["dq"] * q), np.sum(do * o), rtol=1e-11)


# ---------------------------------------------------------------- I12: finite differences
@pytest.mark.parametrize("T,D", [(1, 3), (5, 3), (17, 8), (67, 3)])
def test_finite_difference_gradients(T, D):
    q, k, v, g, beta, h0 = rand_case(12 + T, T=T, Dk=D, Dv=D, unit_k=False, decay=0.5)
    rng = np.random.default_rng(120 + T)
    do, dhT = rng.standard_normal(v.shape), rng.standard_normal(h0.shape)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)

    def loss(a):
        o, hT = ref.fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], 0.45, a["h0"])
        return np.sum(o * do) + np.sum(hT * dhT)

    gr = ref.bwd(q, k, v, g, beta, 0.45, do, h0, dhT)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")
    eps = 1e-6
    for name, gname in names.items():
        flat_idx = rng.choice(args[name].size, size=min(12, args[name].size), replace=False)
        for fi in flat_idx:
            idx = np.unravel_index(fi, args[name].shape)
            ap = {key: val.copy() for key, val in args.items()}
            am = {key: val.copy() for key, val in args.items()}
            ap[name][idx] += eps
            am[name][idx] -= eps
            fd = (loss(ap) - loss(am)) / (2 * eps)
            an = gr[gname][idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, idx, fd, an)


# ---------------------------------------------------------------- oracle sanity on planted mistakes
def test_pins_catch_a_transposed_initial_state():
    """The beta = 0 pin distinguishes h0 from h0^T, so an orientation mix-up in
    the oracle's state import would fail it."""
    q, k, v, g, beta, h0 = rand_case(13, T=3, Dk=4, Dv=4)
    beta[:] = 0.0
    o, _ = ref.fwd(q, k, v, g, beta, 1.0, h0)
    o_t, _ = ref.fwd(q, k, v, g, beta, 1.0, np.swapaxes(h0, -1, -2).copy())
    assert relerr(o_t, o) > 1e-3


def test_chunk_t_is_the_forward_chunk_matrix():
    """chunked.chunk_t returns the T that chunked.fwd uses (pinned to the token
    recurrence above): with a zero initial state, one chunk's end state is
    K~^T T diag(beta) V, compared here with the recurrence's hT; short chunks are
    completed with the identity."""
    q, k, v, g, beta, _ = rand_case(9, B=1, T=70, Dk=5, Dv=4)
    C = 16
    ts = chunked.chunk_t(k, g, beta, C=C)
    assert ts.shape == (5, 2, C, C)
    for c in range(5):
        t0, t1 = 16 * c, min(16 * c + 16, 70)
        n = t1 - t0
        _, hT = ref.fwd(q[:, t0:t1], k[:, t0:t1], v[:, t0:t1], g[:, t0:t1], beta[:, t0:t1], 0.6)
        for hh in range(2):
            K, V = k[0, t0:t1, hh], v[0, t0:t1, hh]
            gam = np.cumsum(g[0, t0:t1, hh])
            Kt = np.exp(gam[-1] - gam)[:, None] * K
            U = ts[c, hh, :n, :n] @ (beta[0, t0:t1, hh][:, None] * V)
            assert relerr(Kt.T @ U, hT[0, hh]) < 1e-12
            assert np.array_equal(ts[c, hh, n:, n:], np.eye(C - n))
            assert not np.any(ts[c, hh, :n, n:]) and not np.any(ts[c, hh, n:, :n])


def test_chunk_u_advances_the_recurrence():
    """chunked.chunk_u gives, for every chunk, the state update of the token
    recurrence: h_end = exp(G_last) h_start + K~^T U (h from ref.fwd on the
    prefixes), with a nonzero initial state; short chunks are zero-padded."""
    q, k, v, g, beta, h0 = rand_case(10, B=1, T=45, Dk=5, Dv=4)
    C = 16
    us = chunked.chunk_u(k, v, g, beta, h0, C=C)
    assert us.shape == (3, 2, C, 4)
    sl = lambda a, t: a[:, :t]
    for c in range(3):
        t0, t1 = C * c, min(C * c + C, 45)
        h_start = h0 if t0 == 0 else ref.fwd(sl(q, t0), sl(k, t0), sl(v, t0), sl(g, t0), sl(beta, t0), 0.6, h0)[1]
        h_end = ref.fwd(sl(q, t1), sl(k, t1), sl(v, t1), sl(g, t1), sl(beta, t1), 0.6, h0)[1]
        for hh in range(2):
            gam = np.cumsum(g[0, t0:t1, hh])
            Kt = np.exp(gam[-1] - gam)[:, None] * k[0, t0:t1, hh]
            want = np.exp(gam[-1]) * h_start[0, hh] + Kt.T @ us[c, hh, :t1 - t0]
            assert relerr(want, h_end[0, hh]) < 1e-12
        assert not np.any(us[c, :, t1 - t0:])
