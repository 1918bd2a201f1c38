"""Pins of the pre-processing oracle (oracle/prep.py) against facts that do not
depend on it: inverse maps in closed form, invariances, and central finite
differences of the composed forward for every raw input."""
import numpy as np
import pytest

from oracle import prep, ref


def raw_inputs(seed, B=1, T=7, H=2, Dk=4, Dv=3):
    rng = np.random.default_rng(seed)
    return dict(q=rng.standard_normal((B, T, H, Dk)) * 1.7, k=rng.standard_normal((B, T, H, Dk)) * 0.6,
                v=rng.standard_normal((B, T, H, Dv)), g=rng.standard_normal((B, T, H)),
                beta=rng.standard_normal((B, T, H)), h0=0.3 * rng.standard_normal((B, H, Dk, Dv)),
                do=rng.standard_normal((B, T, H, Dv)), dhT=rng.standard_normal((B, H, Dk, Dv)))


def test_gate_logits_invert_in_closed_form():
    """a = log(expm1(x)) gives g = -s x and b = log(beta / (1 - beta)) gives beta back,
    so the pre-processed operator equals the plain one on (g = -s x, beta)."""
    x = raw_inputs(1)
    rng = np.random.default_rng(11)
    decay = rng.uniform(0.02, 0.5, size=x["g"].shape)
    beta = rng.uniform(0.05, 0.95, size=x["g"].shape)
    s = np.array([0.7, 1.9])
    a = np.log(np.expm1(decay))
    b = np.log(beta / (1.0 - beta))
    o1, h1 = prep.fwd(x["q"], x["k"], x["v"], a, b, 0.5, x["h0"], gate_act=True, gate_scale=s)
    o2, h2 = ref.fwd(x["q"], x["k"], x["v"], -s * decay, beta, 0.5, x["h0"])
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(h1 - h2)) < 1e-12


def test_normalisation_is_scale_invariant():
    """Scaling every raw q and k vector by its own positive factor leaves o and hT
    unchanged (up to the 1e-6 guard), and the unit-norm inputs reproduce the plain
    operator."""
    x = raw_inputs(2)
    rng = np.random.default_rng(5)
    cq = rng.uniform(0.5, 4.0, size=x["q"].shape[:-1] + (1,))
    ck = rng.uniform(0.5, 4.0, size=x["k"].shape[:-1] + (1,))
    o1, h1 = prep.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, x["h0"], qk_norm=True)
    o2, h2 = prep.fwd(x["q"] * cq, x["k"] * ck, x["v"], x["g"], x["beta"], 0.5, x["h0"], qk_norm=True)
    assert np.max(np.abs(o1 - o2)) < 1e-5 * np.max(np.abs(o1))
    qn = x["q"] / np.linalg.norm(x["q"], axis=-1, keepdims=True)
    kn = x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True)
    o3, _ = ref.fwd(qn, kn, x["v"], x["g"], x["beta"], 0.5, x["h0"])
    assert np.max(np.abs(o1 - o3)) < 1e-5 * np.max(np.abs(o3))


def test_raw_gradients_are_orthogonal_to_raw_vectors():
    """The output does not depend on the length of a raw q or k vector, so each row
    of dq (dk) is orthogonal to the matching raw row (to the 1e-6 guard)."""
    x = raw_inputs(3)
    d = prep.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, x["do"], x["h0"], x["dhT"], qk_norm=True)
    for name, raw in (("dq", x["q"]), ("dk", x["k"])):
        dots = np.sum(d[name] * raw, axis=-1)
        assert np.max(np.abs(dots)) < 1e-5 * np.max(np.abs(d[name])) * np.max(np.abs(raw)), name


@pytest.mark.parametrize("qk_norm,gate_act", [(True, False), (False, True), (True, True)])
def test_backward_matches_central_differences(qk_norm, gate_act):
    x = raw_inputs(4 + 2 * qk_norm + gate_act)
    s = np.array([0.3, 1.4]) if gate_act else None
    kw = dict(qk_norm=qk_norm, gate_act=gate_act, gate_scale=s)

    def loss(q, k, v, g, beta, h0):
        o, hT = prep.fwd(q, k, v, g, beta, 0.5, h0, **kw)
        return np.sum(o * x["do"]) + np.sum(hT * x["dhT"])

    grads = prep.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, x["do"], x["h0"], x["dhT"], **kw)
    names = ["q", "k", "v", "g", "beta", "h0"]
    gname = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", h0="dh0")
    rng = np.random.default_rng(9)
    eps = 1e-6
    for nm in names:
        base = {n: np.array(x[n], dtype=np.float64) for n in names}
        flat = base[nm].reshape(-1)
        for idx in rng.choice(flat.size, size=min(6, flat.size), replace=False):
            plus = {n: a.copy() for n, a in base.items()}
            minus = {n: a.copy() for n, a in base.items()}
            plus[nm].reshape(-1)[idx] += eps
            minus[nm].reshape(-1)[idx] -= eps
            fd = (loss(**plus) - loss(**minus)) / (2 * eps)
            an = grads[gname[nm]].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (nm, idx, fd, an)
