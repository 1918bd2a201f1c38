"""fp64 numpy evaluation of the chunked (WY/UT) form of the gated delta rule.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It never serves as the
GPU's reference; it exists to check that the chunked algebra -- the
"hardware-friendly algebraic reformulation" the "FlashQLA resource" page
(section 3, "The Three Key Features") says loses no numerical precision --
gives the same numbers as the token recurrence in ``ref``.

Per sequence and head, the tokens are cut into chunks of C rows starting at the
sequence start (the last chunk may be shorter).  Inside one chunk with rows
r, i = 0..C'-1, h = S^T the state at the chunk start:

    gam_r = sum_{i<=r} g_i,  Gam = exp(gam),  D_ri = exp(gam_r - gam_i)
    A  = strict_lower(diag(beta) (K K^T) * D)
    T  = (I + A)^{-1}
    W  = T diag(beta*Gam) K,      Ut = T diag(beta) V
    U  = Ut - W h
    P  = (Q K^T) * D * [i <= r]
    O  = scale (diag(Gam) Q h + P U)
    h' = exp(gam_last) h + Kt^T U,   Kt = diag(exp(gam_last - gam)) K

The backward is the reverse-mode derivative of exactly these lines, chunk by
chunk from the last to the first, with dh' the gradient at the chunk end.
"""
import numpy as np


def _cu(B, T, cu_seqlens):
    if cu_seqlens is None:
        return np.arange(B + 1, dtype=np.int64) * T
    return np.asarray(cu_seqlens, dtype=np.int64)


def _chunk_consts(Kc, g, b):
    gam = np.cumsum(g)
    Gam = np.exp(gam)
    Dm = np.exp(gam[:, None] - gam[None, :])
    Cn = len(g)
    low = np.tril(np.ones((Cn, Cn)), -1)
    A = (b[:, None] * (Kc @ Kc.T) * Dm) * low
    T = np.linalg.inv(np.eye(Cn) + A)
    return gam, Gam, Dm, A, T


def chunk_t(k, g, beta, cu_seqlens=None, C=64):
    """Every chunk's T = (I + A)^{-1} of the lines above, float64 [chunks, H, C, C],
    chunks numbered sequence after sequence.  A short last chunk is completed with
    identity rows and columns (its missing rows carry beta = 0)."""
    k, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, g, beta))
    B, T, H, Dk = k.shape
    cu = _cu(B, T, cu_seqlens)
    kf, gf, bf = k.reshape(B * T, H, Dk), g.reshape(B * T, H), beta.reshape(B * T, H)
    out = []
    for n in range(len(cu) - 1):
        for t0 in range(cu[n], cu[n + 1], C):
            t1 = min(t0 + C, cu[n + 1])
            ts = np.tile(np.eye(C), (H, 1, 1))
            for hh in range(H):
                ts[hh, :t1 - t0, :t1 - t0] = _chunk_consts(kf[t0:t1, hh], gf[t0:t1, hh], bf[t0:t1, hh])[4]
            out.append(ts)
    return np.stack(out) if out else np.zeros((0, H, C, C))


def chunk_u(k, v, g, beta, h0=None, cu_seqlens=None, C=64):
    """Every chunk's U = Ut - W h of the lines above (h the state at the chunk
    start), float64 [chunks, H, C, Dv], chunks numbered sequence after sequence;
    a short last chunk's missing rows are zero."""
    k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, v, g, beta))
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    cu = _cu(B, T, cu_seqlens)
    kf, vf = k.reshape(B * T, H, Dk), v.reshape(B * T, H, Dv)
    gf, bf = g.reshape(B * T, H), beta.reshape(B * T, H)
    out = []
    for n in range(len(cu) - 1):
        hs = [np.zeros((Dk, Dv)) if h0 is None else np.array(h0[n, hh], dtype=np.float64) for hh in range(H)]
        for t0 in range(cu[n], cu[n + 1], C):
            t1 = min(t0 + C, cu[n + 1])
            us = np.zeros((H, C, Dv))
            for hh in range(H):
                K, V = kf[t0:t1, hh], vf[t0:t1, hh]
                gc, bc = gf[t0:t1, hh], bf[t0:t1, hh]
                gam, Gam, Dm, A, Tm = _chunk_consts(K, gc, bc)
                U = Tm @ (bc[:, None] * V) - Tm @ ((bc * Gam)[:, None] * K) @ hs[hh]
                us[hh, :t1 - t0] = U
                Kt = np.exp(gam[-1] - gam)[:, None] * K
                hs[hh] = np.exp(gam[-1]) * hs[hh] + Kt.T @ U
            out.append(us)
    return np.stack(out) if out else np.zeros((0, H, C, Dv))


def fwd(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, C=64):
    """Chunked forward; returns (o, hT) in float64 (same shapes as ``ref.fwd``)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    cu = _cu(B, T, cu_seqlens)
    N = len(cu) - 1
    qf, kf, vf = q.reshape(B * T, H, Dk), k.reshape(B * T, H, Dk), v.reshape(B * T, H, Dv)
    gf, bf = g.reshape(B * T, H), beta.reshape(B * T, H)
    o = np.zeros((B * T, H, Dv))
    hT = np.zeros((N, H, Dk, Dv))
    for n in range(N):
        for hh in range(H):
            h = np.zeros((Dk, Dv)) if h0 is None else np.array(h0[n, hh], dtype=np.float64)
            for t0 in range(cu[n], cu[n + 1], C):
                t1 = min(t0 + C, cu[n + 1])
                Q, K, V = qf[t0:t1, hh], kf[t0:t1, hh], vf[t0:t1, hh]
                gc, bc = gf[t0:t1, hh], bf[t0:t1, hh]
                gam, Gam, Dm, A, Tm = _chunk_consts(K, gc, bc)
                W = Tm @ ((bc * Gam)[:, None] * K)
                Ut = Tm @ (bc[:, None] * V)
                U = Ut - W @ h
                P = (Q @ K.T) * Dm * np.tril(np.ones_like(Dm))
                o[t0:t1, hh] = scale * (Gam[:, None] * (Q @ h) + P @ U)
                Kt = np.exp(gam[-1] - gam)[:, None] * K
                h = np.exp(gam[-1]) * h + Kt.T @ U
            hT[n, hh] = h
    return o.reshape(B, T, H, Dv), hT


def bwd(q, k, v, g, beta, scale, do, h0=None, dhT=None, cu_seqlens=None, C=64):
    """Chunked backward; returns dict dq, dk, dv, dg, dbeta, dh0 (float64)."""
    q, k, v, g, beta, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, do))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    cu = _cu(B, T, cu_seqlens)
    N = len(cu) - 1
    R = B * T
    qf, kf, vf, dof = (x.reshape(R, H, -1) for x in (q, k, v, do))
    gf, bf = g.reshape(R, H), beta.reshape(R, H)
    dq, dk, dv = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(vf)
    dg, dbeta = np.zeros_like(gf), np.zeros_like(bf)
    dh0 = np.zeros((N, H, Dk, Dv))
    for n in range(N):
        for hh in range(H):
            starts = list(range(cu[n], cu[n + 1], C))
            # forward replay: state at every chunk start
            hs = []
            h = np.zeros((Dk, Dv)) if h0 is None else np.array(h0[n, hh], dtype=np.float64)
            for t0 in starts:
                t1 = min(t0 + C, cu[n + 1])
                K, V = kf[t0:t1, hh], vf[t0:t1, hh]
                gc, bc = gf[t0:t1, hh], bf[t0:t1, hh]
                gam, Gam, Dm, A, Tm = _chunk_consts(K, gc, bc)
                U = Tm @ (bc[:, None] * V) - Tm @ ((bc * Gam)[:, None] * K) @ h
                hs.append(h)
                h = np.exp(gam[-1]) * h + (np.exp(gam[-1] - gam)[:, None] * K).T @ U
            dhn = np.zeros((Dk, Dv)) if dhT is None else np.array(dhT[n, hh], dtype=np.float64)
            for ci in range(len(starts) - 1, -1, -1):
                t0 = starts[ci]
                t1 = min(t0 + C, cu[n + 1])
                h = hs[ci]
                Q, K, V, dO = qf[t0:t1, hh], kf[t0:t1, hh], vf[t0:t1, hh], dof[t0:t1, hh]
                gc, bc = gf[t0:t1, hh], bf[t0:t1, hh]
                gam, Gam, Dm, A, Tm = _chunk_consts(K, gc, bc)
                Cn = len(gc)
                causal = np.tril(np.ones((Cn, Cn)))
                Mm = Dm * causal
                B1 = (bc * Gam)[:, None] * K
                B2 = bc[:, None] * V
                W = Tm @ B1
                U = Tm @ B2 - W @ h
                P = (Q @ K.T) * Mm
                ek = np.exp(gam[-1] - gam)
                Kt = ek[:, None] * K
                # reverse of O and h'
                GP = scale * (dO @ U.T) * causal
                dU = scale * P.T @ dO + Kt @ dhn
                dh = scale * (Gam[:, None] * Q).T @ dO + np.exp(gam[-1]) * dhn - W.T @ dU
                GW = -dU @ h.T
                XW = Tm.T @ GW
                XU = Tm.T @ dU
                GT = dU @ B2.T + GW @ B1.T
                GA = np.tril(-Tm.T @ GT @ Tm.T, -1)
                E = bc[:, None] * (GA * Dm)
                KK = K @ K.T
                dq[t0:t1, hh] = scale * Gam[:, None] * (dO @ h.T) + (GP * Mm) @ K
                dk[t0:t1, hh] = ((GP * Mm).T @ Q + ek[:, None] * (U @ dhn.T)
                                 + (bc * Gam)[:, None] * XW + (E + E.T) @ K)
                dv[t0:t1, hh] = bc[:, None] * XU
                dbeta[t0:t1, hh] = (np.sum(XU * V, 1) + Gam * np.sum(XW * K, 1)
                                    + np.sum(GA * Dm * KK, 1))
                GPP = GP * P
                GAA = GA * A
                Udh = U @ dhn.T  # row r: dh' u_r
                dgam = (scale * Gam * np.sum(Q * (dO @ h.T), 1)
                        + bc * Gam * np.sum(XW * K, 1)
                        + GPP.sum(1) - GPP.sum(0) + GAA.sum(1) - GAA.sum(0)
                        - ek * np.sum(K * Udh, 1))
                dgam[-1] += np.exp(gam[-1]) * np.sum(h * dhn) + np.sum(ek * np.sum(K * Udh, 1))
                dg[t0:t1, hh] = np.cumsum(dgam[::-1])[::-1]
                dhn = dh
            dh0[n, hh] = dhn
    shp = lambda x, d: x.reshape(B, T, H, d)
    return dict(dq=shp(dq, Dk), dk=shp(dk, Dk), dv=shp(dv, Dv),
                dg=dg.reshape(B, T, H), dbeta=dbeta.reshape(B, T, H), dh0=dh0)
