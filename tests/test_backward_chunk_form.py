"""The chunk-level form of the backward, checked against the oracle's per-token backward.

The backward kernels differentiate the per-token update. A chunked backward (64-token chunks,
products on matrix cores) would instead differentiate the chunk form of the forward: with
Gamma_t the in-chunk cumulative decay, K_G = K e^G, Q_G = Q e^G, K^ = K e^{G_C - G},
A = tril(diag(beta) K_G (K e^-G)^T, -1), T = (I + A)^-1, M = tril(Q_G (K e^-G)^T),
Y = diag(beta)(V - K_G S0), U = T Y, O = s(Q_G S0 + M U), S_C = e^{G_C} S0 + K^T U.
This test writes that backward out in fp64 (one chunk at a time, in reverse) and requires it to
equal recurrence_bwd, so the derivation is pinned before any kernel is built on it."""
import numpy as np
import pytest

from oracle import kda_oracle as ko


def _chunk_bwd(q, k, v, g, beta, do, dht, h0, scale, gmin=-5.0, C=64):
    T, dk = q.shape
    gt = np.maximum(g, gmin)
    live = g > gmin
    bounds = [(c, min(T, c + C)) for c in range(0, T, C)]
    S = h0.copy()
    S0s = []
    for a, b in bounds:
        G = np.cumsum(gt[a:b], axis=0)
        Kg, Kh, Kn = k[a:b] * np.exp(G), k[a:b] * np.exp(G[-1] - G), k[a:b] * np.exp(-G)
        A = np.tril(beta[a:b, None] * (Kg @ Kn.T), -1)
        U = np.linalg.inv(np.eye(b - a) + A) @ (beta[a:b, None] * (v[a:b] - Kg @ S))
        S0s.append(S.copy())
        S = np.exp(G[-1])[:, None] * S + Kh.T @ U
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g),
                                              ("dbeta", beta))}
    dS = dht.copy()
    for ci in reversed(range(len(bounds))):
        a, b = bounds[ci]
        S0, L = S0s[ci], b - a
        G = np.cumsum(gt[a:b], axis=0)
        GC, Gam = G[-1], np.exp(G)
        Kg, Qg = k[a:b] * Gam, q[a:b] * Gam
        Kh, Kn = k[a:b] * np.exp(GC - G), k[a:b] * np.exp(-G)
        B = Kg @ Kn.T                              # k_t . k_s e^{G_t - G_s}
        Tm = np.linalg.inv(np.eye(L) + np.tril(beta[a:b, None] * B, -1))
        M = np.tril(Qg @ Kn.T)
        X0 = v[a:b] - Kg @ S0
        Y = beta[a:b, None] * X0
        U = Tm @ Y
        dO = do[a:b]
        dU = scale * M.T @ dO + Kh @ dS
        dY = Tm.T @ dU
        dA = np.tril(-Tm.T @ (dU @ Y.T) @ Tm.T, -1)
        dM = np.tril(scale * dO @ U.T)
        out["dv"][a:b] = beta[a:b, None] * dY
        out["dbeta"][a:b] = np.sum(X0 * dY, 1) + np.sum(dA * B, 1)
        E = np.exp(G[:, None, :] - G[None, :, :])  # [t, s, c], used for s <= t
        W = dA * beta[a:b, None]
        dq_m = np.einsum("ts,sc,tsc->tc", dM, k[a:b], E)
        dk_mkey = np.einsum("ts,tc,tsc->sc", dM, q[a:b], E)
        dk_aq = np.einsum("ts,sc,tsc->tc", W, k[a:b], E)
        dk_akey = np.einsum("ts,tc,tsc->sc", W, k[a:b], E)
        dk_kg = -(beta[a:b, None] * dY) @ S0.T * Gam
        dk_kh = (U @ dS.T) * np.exp(GC - G)
        dq = scale * dO @ S0.T * Gam + dq_m
        out["dq"][a:b] = dq
        out["dk"][a:b] = dk_kg + dk_aq + dk_akey + dk_mkey + dk_kh
        dG = q[a:b] * dq + k[a:b] * (dk_kg + dk_aq) - k[a:b] * (dk_akey + dk_mkey + dk_kh)
        dG[-1] += np.sum(k[a:b] * dk_kh, 0) + np.sum(dS * (np.exp(GC)[:, None] * S0), 1)
        out["dg"][a:b] = np.cumsum(dG[::-1], axis=0)[::-1] * live[a:b]
        dS = scale * Qg.T @ dO + np.exp(GC)[:, None] * dS - Kg.T @ (beta[a:b, None] * dY)
    out["dh0"] = dS
    return out


@pytest.mark.parametrize("T,d,stress", [(150, 16, False), (200, 32, True), (64, 8, False),
                                        (65, 8, True)])
def test_chunk_form_equals_per_token_backward(T, d, stress):
    rng = np.random.default_rng(T + d)
    unit = lambda x: x / np.linalg.norm(x, axis=1, keepdims=True)
    q, k = unit(rng.standard_normal((T, d))), unit(rng.standard_normal((T, d)))
    v = rng.standard_normal((T, d))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    graw = rng.standard_normal((T, d))
    g = -np.log1p(np.exp(10 * graw if stress else graw))
    if not stress:
        g = np.maximum(g, -5.0)
    do, dht = rng.standard_normal((T, d)), rng.standard_normal((d, d))
    h0 = 0.1 * rng.standard_normal((d, d))
    ref = ko.recurrence_bwd(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                            do[:, None], dht=dht[None, None], h0=h0[None, None], scale=0.8)
    got = _chunk_bwd(q, k, v, g, beta, do, dht, h0, 0.8)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        r = ref[n][0, 0] if n == "dh0" else ref[n][:, 0]
        err = np.abs(got[n] - r).max() / np.sqrt(np.mean(r * r))
        assert err < 1e-10, (n, err)
