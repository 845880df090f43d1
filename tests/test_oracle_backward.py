"""Pins of the oracle's backward (recurrence_bwd): the gradients of the forward definition
(recurrence_fwd, itself pinned elsewhere) checked against central finite differences of that
forward, against the closed forms of the beta = 0 special case, and for the flat floor."""
import numpy as np

from oracle import kda_oracle as ko


def _inputs(seed, T=7, H=2, dk=3, dv=2, N=2, g_lo=-2.0, g_min=-1.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(g_lo, 0.0, (T, H, dk))
    # keep clear of the floor's kink so that the differences are one-sided on neither side
    g = np.where(np.abs(g - g_min) < 0.05, g_min + 0.1, g)
    beta = rng.uniform(0.1, 0.9, (T, H))
    h0 = 0.5 * rng.standard_normal((N, H, dk, dv))
    Wo = rng.standard_normal((T, H, dv))          # dL/do
    Wh = rng.standard_normal((N, H, dk, dv))      # dL/dht
    return q, k, v, g, beta, h0, Wo, Wh


def test_gradients_match_central_differences():
    """Two packed sequences (lengths 3 and 4), the floor active on part of g: every gradient
    of L = <o, Wo> + <ht, Wh> equals its central difference through the forward oracle."""
    cu = [0, 3, 7]
    g_min, scale, eps = -1.5, 0.7, 1e-6
    q, k, v, g, beta, h0, Wo, Wh = _inputs(3, g_min=g_min)
    assert (g < g_min).any() and (g > g_min).any()
    args = dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0)

    def loss(a):
        o, ht = ko.recurrence_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], h0=a["h0"],
                                  cu_seqlens=cu, scale=scale, g_min=g_min)
        return np.sum(o * Wo) + np.sum(ht * Wh)

    grads = ko.recurrence_bwd(q, k, v, g, beta, Wo, dht=Wh, h0=h0, cu_seqlens=cu, scale=scale,
                              g_min=g_min)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                      ("h0", "dh0")):
        x = args[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            plus, minus = dict(args), dict(args)
            plus[name] = x.copy()
            plus[name][idx] += eps
            minus[name] = x.copy()
            minus[name][idx] -= eps
            num[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        np.testing.assert_allclose(grads[key], num, rtol=1e-6, atol=1e-7, err_msg=key)


def test_beta_zero_closed_forms():
    """beta = 0: no correction, S_t = diag(A_t) h0 with A_t the running product of the decays,
    so dq_t = scale diag(A_t) h0 do_t, dh0 = sum_t scale diag(A_t) q_t do_t^T + diag(A_T) dht,
    and v and k receive no gradient."""
    q, k, v, g, _, h0, Wo, Wh = _inputs(5, N=1)
    T = q.shape[0]
    beta = np.zeros((T, q.shape[1]))
    scale, g_min = 1.3, -5.0
    grads = ko.recurrence_bwd(q, k, v, g, beta, Wo, dht=Wh, h0=h0, scale=scale, g_min=g_min)
    A = np.cumprod(np.exp(np.maximum(g, g_min)), axis=0)          # [T, H, d_k]
    dq = scale * np.einsum("thk,hkv,thv->thk", A, h0[0], Wo)
    dh0 = (scale * np.einsum("thk,thk,thv->hkv", A, q, Wo) + A[-1][:, :, None] * Wh[0])
    np.testing.assert_allclose(grads["dq"], dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(grads["dh0"][0], dh0, rtol=1e-12, atol=1e-12)
    assert not grads["dv"].any() and not grads["dk"].any()


def test_floored_decay_gets_no_gradient():
    """Where g_t lies below the floor the decay does not depend on it."""
    q, k, v, g, beta, h0, Wo, Wh = _inputs(7, N=1, g_lo=-4.0, g_min=-1.0)
    grads = ko.recurrence_bwd(q, k, v, g, beta, Wo, dht=Wh, h0=h0, g_min=-1.0)
    below = g < -1.0
    assert below.any()
    assert np.all(grads["dg"][below] == 0.0)
    assert np.all(grads["dg"][~below] != 0.0)
