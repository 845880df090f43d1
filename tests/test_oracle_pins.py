"""Pins for the CPU oracle: every check here compares it with something other than itself
(values printed on the pages, closed forms, brute force, invariants, library routines on
special cases). CPU only."""

import json
import math
import os

import numpy as np
import pytest

from oracle import c_recurrence_fwd
from oracle import kda_oracle as ko

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_inputs(rng, T, H, dk, dv, g_scale=1.0, floor=True):
    q = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0.0, g_scale * rng.standard_normal((T, H, dk)))
    if floor:
        g = np.maximum(g, -5.0)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


# ------------------------------------------------------------------ worked examples (pages)
def test_worked_example_segment_composition():
    """AMD blog section 5: 'halve and add 2' then 'halve and add 1' = 'quarter plus 2'."""
    gold = _golden("segment_composition_scalar.json")
    toks = gold["tokens"]
    k = np.array([[t["k"]] for t in toks])
    v = np.array([[t["v"]] for t in toks])
    g = np.array([[t["g"]] for t in toks])
    beta = np.array([t["beta"] for t in toks])
    # each single token is the printed map s -> a s + b
    for t, (a, b) in enumerate(gold["maps"]):
        P, Q = ko.segment_transition(k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1])
        assert P[0, 0] == a and Q[0, 0] == b
    # the two-token segment is the composed map, computed without the incoming state
    P, Q = ko.segment_transition(k, v, g, beta)
    assert (P[0, 0], Q[0, 0]) == tuple(gold["composed"])
    # and the token-by-token recurrence from any entering state lands on s/4 + 2
    for s0 in [-3.0, 0.0, 1.5, 8.0]:
        _, ht = ko.recurrence_fwd(k[:, None, :], k[:, None, :], v[:, None, :], g[:, None, :],
                                  beta[:, None], h0=np.array([[[[s0]]]]))
        assert ht[0, 0, 0, 0] == gold["composed"][0] * s0 + gold["composed"][1]
    # composing the two single-token summaries with the ordered scan gives the same result
    Ps, Qs = zip(*[ko.segment_transition(k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1])
                   for t in range(2)])
    states = ko.segment_scan(np.array([[8.0]]), Ps, Qs)
    assert states[-1][0, 0] == 0.25 * 8.0 + 2.0


def test_worked_example_dependency_inverse():
    """Nota técnica: dependency coefficients 1/4, 1/8 and the inverse's -1/4, -1/16."""
    gold = _golden("ut_inverse_scalar.json")
    k = np.array(gold["tokens"]["k"])[:, None]
    beta = np.array(gold["tokens"]["beta"])
    g = np.full((3, 1), math.log(0.5))
    A = ko.chunk_dependency_matrix(k, g, beta)
    np.testing.assert_allclose(A, np.array(gold["dependency"]), rtol=0, atol=1e-15)
    # exact A gives the exact printed inverse (all entries are dyadic)
    T = ko.unit_lower_inverse(np.array(gold["dependency"]))
    assert np.array_equal(T, np.array(gold["inverse"]))
    # the bottom-left entry is the direct effect plus the path through position two
    assert T[2, 0] == gold["direct_effect_1_on_3"] + gold["path_via_2"]
    # a library inverse of I + A agrees
    np.testing.assert_allclose(np.linalg.inv(np.eye(3) + np.array(gold["dependency"])), T,
                               rtol=0, atol=1e-15)
    # and the chunk form built on it reproduces the token-by-token run of that example
    rng = np.random.default_rng(5)
    v = rng.standard_normal((3, 1, 2))
    q = np.ones((3, 1, 1))
    o_ref, s_ref = ko.recurrence_fwd(q, k[:, None, :], v, g[:, None, :], beta[:, None])
    o_ch, s_ch = ko.chunked_fwd(q, k[:, None, :], v, g[:, None, :], beta[:, None], chunk=3)
    np.testing.assert_allclose(o_ch, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(s_ch[0], s_ref[0, 0], rtol=0, atol=1e-14)


def test_bf16_rounding_example_fixture():
    """Nota técnica table: 256.5 rounds to 256 in bf16, the fp32 difference keeps 0.5. Pins
    the fixture the GPU precision test uses (torch's RNE cast)."""
    torch = pytest.importorskip("torch")
    gold = _golden("bf16_rounding_example.json")
    a32 = torch.tensor(gold["a"], dtype=torch.float32)
    b32 = torch.tensor(gold["b"], dtype=torch.float32)
    assert float(a32 - b32) == gold["fp32_result"]
    assert float(a32.to(torch.bfloat16).float() - b32) == gold["bf16_first_result"]


# ------------------------------------------------------------------ closed forms
def test_closed_form_beta_zero_with_floor():
    """beta = 0: pure per-channel decay, S_T = diag(exp(sum max(g, g_min))) S_0 and
    o_t = scale (diag(exp(sum_{s<=t} max(g_s, g_min))) S_0)^T q_t. Raw g scaled by 10 so the
    floor at -5 bites."""
    rng = np.random.default_rng(1)
    T, H, dk, dv = 23, 2, 6, 5
    q, k, v, g, _ = _rand_inputs(rng, T, H, dk, dv, g_scale=10.0, floor=False)
    assert (g < -5.0).any()
    beta = np.zeros((T, H))
    h0 = rng.standard_normal((1, H, dk, dv))
    scale = 0.75
    o, ht = ko.recurrence_fwd(q, k, v, g, beta, h0=h0, scale=scale)
    G = np.cumsum(np.clip(g, -5.0, None), axis=0)          # [T, H, dk]
    for t in range(T):
        St = np.exp(G[t])[:, :, None] * h0[0]
        np.testing.assert_allclose(o[t], scale * np.einsum("hkv,hk->hv", St, q[t]),
                                   rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ht[0], np.exp(G[-1])[:, :, None] * h0[0], rtol=1e-12, atol=0)


def test_closed_form_overwrite_orthonormal_keys():
    """g = 0, beta = 1, orthonormal keys: every token overwrites its key's slot,
    S_t^T k_t = v_t, and S_T = (I - K^T K) S_0 + K^T V."""
    rng = np.random.default_rng(2)
    dk, dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:, :T].T                                   # T orthonormal rows
    V = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((dk, dv))
    o, ht = ko.recurrence_fwd(K[:, None, :], K[:, None, :], V[:, None, :],
                              np.zeros((T, 1, dk)), np.ones((T, 1)), h0=S0[None, None])
    # reading out with q = k_t right after token t returns exactly v_t
    np.testing.assert_allclose(o[:, 0], V, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], (np.eye(dk) - K.T @ K) @ S0 + K.T @ V, rtol=0,
                               atol=1e-12)


def test_brute_force_small():
    """T <= 16: the running recurrence equals the explicit expansion over transition
    products."""
    rng = np.random.default_rng(3)
    for T, dk, dv in [(1, 3, 2), (7, 4, 3), (16, 5, 4)]:
        q, k, v, g, beta = _rand_inputs(rng, T, 1, dk, dv, g_scale=3.0)
        h0 = rng.standard_normal((dk, dv))
        o, ht = ko.recurrence_fwd(q, k, v, g, beta, h0=h0[None, None], scale=0.5)
        ob, Sb = ko.brute_force_fwd(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], h0, scale=0.5)
        np.testing.assert_allclose(o[:, 0], ob, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht[0, 0], Sb, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ chunk and segment algebra
@pytest.mark.parametrize("T,chunk", [(64, 64), (150, 64), (37, 16), (200, 32)])
def test_chunked_equals_per_token(T, chunk):
    rng = np.random.default_rng(T + chunk)
    H, dk, dv = 2, 8, 6
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=2.0)
    h0 = 0.3 * rng.standard_normal((1, H, dk, dv))
    o, ht = ko.recurrence_fwd(q, k, v, g, beta, h0=h0, scale=0.9)
    oc, hc = ko.chunked_fwd(q, k, v, g, beta, h0=h0[0], scale=0.9, chunk=chunk)
    np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hc, ht[0], rtol=1e-11, atol=1e-12)


def test_chunked_with_floor_stress():
    rng = np.random.default_rng(11)
    T, H, dk, dv = 96, 1, 6, 4
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=10.0, floor=False)
    o, ht = ko.recurrence_fwd(q, k, v, g, beta)
    oc, hc = ko.chunked_fwd(q, k, v, g, beta, chunk=64)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hc, ht[0], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("bounds", [[0, 40, 90], [0, 10, 20, 30, 60, 90], [0, 89, 90]])
def test_segment_composition_equals_full_run(bounds):
    rng = np.random.default_rng(len(bounds))
    T, dk, dv = 90, 5, 4
    q, k, v, g, beta = _rand_inputs(rng, T, 1, dk, dv, g_scale=1.5)
    h0 = rng.standard_normal((dk, dv))
    bounds = bounds + [T] if bounds[-1] != T else bounds
    Ps, Qs = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        P, Q = ko.segment_transition(k[a:b, 0], v[a:b, 0], g[a:b, 0], beta[a:b, 0])
        Ps.append(P)
        Qs.append(Q)
    states = ko.segment_scan(h0, Ps, Qs)
    # every segment's entering state equals the token-by-token state at that boundary
    for j, a in enumerate(bounds):
        if a == 0:
            np.testing.assert_allclose(states[j], h0)
            continue
        _, ht = ko.recurrence_fwd(q[:a], k[:a], v[:a], g[:a], beta[:a], h0=h0[None, None])
        np.testing.assert_allclose(states[j], ht[0, 0], rtol=1e-11, atol=1e-12)
    # replaying each segment from its entering state reproduces the full outputs
    o_full, _ = ko.recurrence_fwd(q, k, v, g, beta, h0=h0[None, None])
    for j, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        o_seg, _ = ko.recurrence_fwd(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                     h0=states[j][None, None])
        np.testing.assert_allclose(o_seg, o_full[a:b], rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------ invariants
def test_linearity_in_state_and_values():
    rng = np.random.default_rng(4)
    T, H, dk, dv = 30, 2, 5, 4
    q, k, v1, g, beta = _rand_inputs(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s1 = rng.standard_normal((1, H, dk, dv))
    s2 = rng.standard_normal((1, H, dk, dv))
    o1, h1 = ko.recurrence_fwd(q, k, v1, g, beta, h0=s1)
    o2, h2 = ko.recurrence_fwd(q, k, v2, g, beta, h0=s2)
    o3, h3 = ko.recurrence_fwd(q, k, 2.0 * v1 - v2, g, beta, h0=2.0 * s1 - s2)
    np.testing.assert_allclose(o3, 2.0 * o1 - o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h3, 2.0 * h1 - h2, rtol=1e-11, atol=1e-12)


def test_heads_and_value_columns_independent():
    rng = np.random.default_rng(6)
    T, H, dk, dv = 25, 3, 5, 6
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    h0 = rng.standard_normal((1, H, dk, dv))
    o, ht = ko.recurrence_fwd(q, k, v, g, beta, h0=h0)
    for h in range(H):
        oh, hh = ko.recurrence_fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], g[:, h:h + 1],
                                   beta[:, h:h + 1], h0=h0[:, h:h + 1])
        np.testing.assert_allclose(oh[:, 0], o[:, h], rtol=1e-13, atol=1e-14)
    cols = [1, 4]
    oc, hc = ko.recurrence_fwd(q, k, v[..., cols], g, beta, h0=h0[..., cols])
    np.testing.assert_allclose(oc, o[..., cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(hc, ht[..., cols], rtol=1e-13, atol=1e-14)


def test_varlen_packing_equals_separate_runs_and_empty_sequence():
    rng = np.random.default_rng(7)
    lengths = [13, 0, 40, 1, 7]
    T, H, dk, dv = sum(lengths), 2, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    h0 = rng.standard_normal((len(lengths), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, ht = ko.recurrence_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu)
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        on, hn = ko.recurrence_fwd(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], h0=h0[n:n + 1])
        np.testing.assert_allclose(o[a:b], on, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(ht[n], hn[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(ht[1], h0[1])          # length 0 leaves h0 unchanged


def test_token_transition_is_a_contraction():
    """For unit k, beta in [0, 1] and g <= 0, ||(I - beta k k^T) diag(e^g)||_2 <= 1."""
    rng = np.random.default_rng(8)
    for _ in range(200):
        k = rng.standard_normal(7)
        k /= np.linalg.norm(k)
        A = ko.token_transition(k, -np.abs(rng.standard_normal(7)) * 3, rng.uniform(0, 1))
        assert np.linalg.norm(A, 2) <= 1.0 + 1e-12


def test_state_column_energy_bound():
    """Unit keys, beta in [0, 1], g <= 0: one token adds at most v_c^2 to the squared norm of
    state column c, so ||S_T[:, c]||^2 <= ||S_0[:, c]||^2 + sum_t v_{t,c}^2 (with the decay
    first, the correction e = v - S'^T k changes the component along k only). Equality holds
    for beta = 1, g = 0, keys orthonormal to each other and to the entering columns."""
    rng = np.random.default_rng(12)
    dk, dv = 12, 5
    for trial in range(6):
        T = 40 + 13 * trial
        q, k, v, g, beta = _rand_inputs(rng, T, 1, dk, dv, g_scale=0.5)
        g *= 0.05                     # decays near 1: the state keeps most of its past
        v *= 1.0 + 3.0 * rng.random((T, 1, 1))
        h0 = rng.standard_normal((1, 1, dk, dv))
        for L in (1, T // 3, T):
            _, ht = ko.recurrence_fwd(q[:L], k[:L], v[:L], g[:L], beta[:L], h0=h0)
            lhs = np.sum(ht[0, 0] ** 2, axis=0)
            rhs = np.sum(h0[0, 0] ** 2, axis=0) + np.sum(v[:L, 0] ** 2, axis=0)
            assert np.all(lhs <= rhs * (1 + 1e-12)), (trial, L, lhs, rhs)
    # equality case: orthonormal keys, overwrite, zero entering state
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:, :8].T
    V = rng.standard_normal((8, dv))
    _, ht = ko.recurrence_fwd(K[:, None], K[:, None], V[:, None], np.zeros((8, 1, dk)),
                              np.ones((8, 1)))
    np.testing.assert_allclose(np.sum(ht[0, 0] ** 2, axis=0), np.sum(V ** 2, axis=0),
                               rtol=1e-12)


# ------------------------------------------------------------------ C oracle twin
@pytest.mark.parametrize("shape", [(256, 2, 64, 64), (70, 3, 16, 24)])
def test_c_oracle_matches_numpy(shape):
    T, H, dk, dv = shape
    rng = np.random.default_rng(T)
    q, k, v, g, beta = [x.astype(np.float32) for x in _rand_inputs(rng, T, H, dk, dv)]
    lengths = [T // 3, 0, T - T // 3]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    h0 = (0.1 * rng.standard_normal((3, H, dk, dv))).astype(np.float32)
    o, ht = ko.recurrence_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu, scale=0.6)
    oc, hc = c_recurrence_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu, scale=0.6, col_block=16)
    np.testing.assert_allclose(oc, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(hc, ht, rtol=1e-12, atol=1e-13)
    oc0, _ = c_recurrence_fwd(q, k, v, g, beta, h0=None, cu_seqlens=cu, col_block=7)
    o0, _ = ko.recurrence_fwd(q, k, v, g, beta, h0=None, cu_seqlens=cu)
    np.testing.assert_allclose(oc0, o0, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ decode pieces
def test_decode_elementary_functions():
    assert ko.silu(0.0) == 0.0
    assert ko.sigmoid(0.0) == 0.5
    assert ko.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-15)
    np.testing.assert_allclose(ko.softplus(np.array([-40.0, 40.0])), [math.exp(-40.0), 40.0],
                               rtol=1e-12)
    np.testing.assert_allclose(ko.silu(np.array([3.0])), [3.0 / (1.0 + math.exp(-3.0))])


def test_causal_conv_matches_numpy_convolve():
    """The depthwise causal window equals np.convolve over the channel's history."""
    rng = np.random.default_rng(9)
    C, W, n = 5, 4, 12
    w = rng.standard_normal((C, W))
    xs = rng.standard_normal((n, C))
    tail = rng.standard_normal((C, W - 1))
    hist = np.concatenate([tail.T, xs], axis=0)          # oldest first
    for t in range(n):
        y, tail = ko.causal_conv_window(tail, xs[t], w)
        for c in range(C):
            full = np.convolve(hist[:, c], w[c, ::-1], mode="valid")
            assert y[c] == pytest.approx(full[t], rel=1e-12, abs=1e-12)
    # delta taps pick the current input or the oldest tail entry
    y, _ = ko.causal_conv_window(tail, xs[0], np.eye(W)[None, W - 1].repeat(C, 0))
    np.testing.assert_array_equal(y, xs[0])
    y, _ = ko.causal_conv_window(tail, xs[0], np.eye(W)[None, 0].repeat(C, 0))
    np.testing.assert_array_equal(y, tail[:, 0])


def _decode_workload(rng, R, H, dk, dv, W, n_new, window):
    def win(slots, z):
        d = dict(q=rng.standard_normal((R, slots, H, dk)), k=rng.standard_normal((R, slots, H, dk)),
                 v=rng.standard_normal((R, slots, H, dv)), g=rng.standard_normal((R, slots, H, dk)),
                 beta=rng.standard_normal((R, slots, H)))
        d["z"] = rng.standard_normal((R, slots, H, dv)) if z else None
        return d
    return dict(prev=win(window, False), new=win(n_new, True),
                conv_w=0.5 * rng.standard_normal((H, 2 * dk + dv, W)),
                norm_w=1 + 0.1 * rng.standard_normal(dv),
                state=0.1 * rng.standard_normal((R, H, dk, dv)),
                tail=rng.standard_normal((R, H, 2 * dk + dv, W - 1)))


def _preprocess(tail, raw, conv_w, dk, act, eps=1e-6):
    """Independent restatement of the input stage for a list of tokens of one head, using
    np.convolve over the whole history (oldest tail entry first)."""
    hist = np.concatenate([tail.T, raw], axis=0)
    C, W = conv_w.shape
    y = np.stack([np.convolve(hist[:, c], conv_w[c, ::-1], mode="valid") for c in range(C)], 1)
    if act:
        y = y / (1 + np.exp(-y))
    q, k, v = y[:, :dk], y[:, dk:2 * dk], y[:, 2 * dk:]
    q = q / np.sqrt((q * q).sum(1, keepdims=True) + eps)
    k = k / np.sqrt((k * k).sum(1, keepdims=True) + eps)
    return q, k, v


def test_decode_single_token_is_one_recurrence_step():
    """n_acc = 0, n_new = 1: the fused token equals convolution + norms + gates followed by
    one step of the prefill recurrence, then the gated RMSNorm."""
    rng = np.random.default_rng(10)
    R, H, dk, dv, W = 2, 2, 6, 5, 4
    wl = _decode_workload(rng, R, H, dk, dv, W, 1, 8)
    out = ko.decode_replay(wl["state"], wl["tail"], np.zeros(R, int), wl["prev"], wl["new"],
                           wl["conv_w"], wl["norm_w"], scale=0.7)
    for r in range(R):
        for h in range(H):
            raw = np.concatenate([wl["new"]["q"][r, :1, h], wl["new"]["k"][r, :1, h],
                                  wl["new"]["v"][r, :1, h]], 1)
            q, k, v = _preprocess(wl["tail"][r, h], raw, wl["conv_w"][h], dk, act=1)
            g = np.maximum(-np.logaddexp(0, wl["new"]["g"][r, :1, h]), -5.0)
            beta = 1 / (1 + np.exp(-wl["new"]["beta"][r, :1, h]))
            o, ht = ko.recurrence_fwd(q[:, None], k[:, None], v[:, None], g[:, None],
                                      beta[:, None], h0=wl["state"][r, h][None, None], scale=0.7)
            o = o[0, 0]
            rms = np.sqrt(np.mean(o * o) + 1e-6)
            gate = 1 / (1 + np.exp(-wl["new"]["z"][r, 0, h]))
            np.testing.assert_allclose(out["o"][r, 0, h], o / rms * wl["norm_w"] * gate,
                                       rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(out["state"][r, h], ht[0, 0], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(out["state_acc"][r, h], wl["state"][r, h])


def test_decode_speculative_stream_is_lossless():
    """Several verify steps with random acceptance: the committed state after each step equals
    the plain recurrence over the committed tokens (bonus tokens and accepted drafts, in
    order), and the replayed state equals the state after the accepted drafts."""
    rng = np.random.default_rng(12)
    R, H, dk, dv, W, n_new = 2, 1, 5, 4, 4, 4
    wl = _decode_workload(rng, R, H, dk, dv, W, n_new, n_new)
    state, tail = wl["state"].copy(), wl["tail"].copy()
    prev = wl["prev"]
    n_acc = np.zeros(R, int)
    committed = [[] for _ in range(R)]                    # raw tokens in commit order
    for step in range(4):
        new = _decode_workload(rng, R, H, dk, dv, W, n_new, n_new)["new"]
        out = ko.decode_replay(state, tail, n_acc, prev, new, wl["conv_w"], wl["norm_w"])
        for r in range(R):
            for j in range(1, n_acc[r] + 1):
                committed[r].append({n: prev[n][r, j, 0] for n in ("q", "k", "v", "g", "beta")})
            n_before_bonus = len(committed[r])
            committed[r].append({n: new[n][r, 0, 0] for n in ("q", "k", "v", "g", "beta")})
            toks = committed[r]
            raw = np.stack([np.concatenate([t["q"], t["k"], t["v"]]) for t in toks])
            q, k, v = _preprocess(wl["tail"][r, 0], raw, wl["conv_w"][0], dk, act=1)
            g = np.maximum(-np.logaddexp(0, np.stack([t["g"] for t in toks])), -5.0)
            beta = 1 / (1 + np.exp(-np.array([t["beta"] for t in toks])))
            _, h_all = ko.recurrence_fwd(q[:, None], k[:, None], v[:, None], g[:, None],
                                         beta[:, None], h0=wl["state"][r, 0][None, None])
            np.testing.assert_allclose(out["state"][r, 0], h_all[0, 0], rtol=1e-10, atol=1e-12)
            _, h_acc = ko.recurrence_fwd(q[:n_before_bonus, None], k[:n_before_bonus, None],
                                         v[:n_before_bonus, None], g[:n_before_bonus, None],
                                         beta[:n_before_bonus, None],
                                         h0=wl["state"][r, 0][None, None])
            np.testing.assert_allclose(out["state_acc"][r, 0], h_acc[0, 0], rtol=1e-10,
                                       atol=1e-12)
        state, tail = out["state"], out["conv_tail"]
        prev = new
        n_acc = rng.integers(0, n_new, R)


def test_decode_output_norm_unit_rms():
    """With unit norm weights and a saturated gate the output has RMS 1 (eps -> 0)."""
    rng = np.random.default_rng(13)
    R, H, dk, dv, W = 1, 1, 4, 6, 4
    wl = _decode_workload(rng, R, H, dk, dv, W, 2, 2)
    wl["new"]["z"][:] = 60.0
    out = ko.decode_replay(wl["state"], wl["tail"], np.zeros(R, int), wl["prev"], wl["new"],
                           wl["conv_w"], np.ones(dv), eps_rms=0.0)
    rms = np.sqrt(np.mean(out["o"] ** 2, axis=-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-12)


def test_raw_prefill_matches_decode_token_steps():
    """The raw prefill's token stage is the decode's: running decode_token (no output) over
    the same tokens from the same state and tail gives the same final state and tail."""
    rng = np.random.default_rng(91)
    T, H, dk, dv, W = 9, 2, 8, 8, 4
    q, k, g = (rng.standard_normal((T, H, dk)) for _ in range(3))
    v = rng.standard_normal((T, H, dv))
    beta = rng.standard_normal((T, H))
    conv_w = 0.5 * rng.standard_normal((H, 2 * dk + dv, W))
    tail = rng.standard_normal((1, H, 2 * dk + dv, W - 1))
    h0 = 0.1 * rng.standard_normal((1, H, dk, dv))
    for act in (0, 1):
        _, ht, tail_out = ko.prefill_raw_fwd(q, k, v, g, beta, conv_w, conv_tail=tail, h0=h0,
                                             act=act)
        for h in range(H):
            S, tl = h0[0, h].copy(), tail[0, h].copy()
            for t in range(T):
                x = dict(q=q[t, h], k=k[t, h], v=v[t, h], g=g[t, h], beta=beta[t, h])
                S, tl, _ = ko.decode_token(S, tl, x, conv_w[h], np.ones(dv), 1.0, -5.0, 1e-6,
                                           1e-6, act, output=False)
            np.testing.assert_allclose(ht[0, h], S, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(tail_out[0, h], tl, rtol=0, atol=0)


def test_raw_prefill_tail_of_short_sequences():
    """A sequence shorter than the tail keeps the older entering-tail entries, shifted; an
    empty sequence hands the entering tail through unchanged."""
    rng = np.random.default_rng(92)
    H, dk, dv, W = 1, 4, 4, 4
    lengths = [2, 0, 5]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    raw = [rng.standard_normal((T, H, dk)) for _ in range(3)]
    v = rng.standard_normal((T, H, dv))
    beta = rng.standard_normal((T, H))
    tail = rng.standard_normal((3, H, 2 * dk + dv, W - 1))
    conv_w = rng.standard_normal((H, 2 * dk + dv, W))
    *_, tail_out = ko.prefill_input_stage(raw[0], raw[1], v, raw[2], beta, conv_w, tail,
                                          cu_seqlens=cu)
    # sequence 0 (two tokens): [old tail slot 2, token 0, token 1]
    np.testing.assert_array_equal(tail_out[0, 0, :dk, 0], tail[0, 0, :dk, 2])
    np.testing.assert_array_equal(tail_out[0, 0, :dk, 1], raw[0][0, 0])
    np.testing.assert_array_equal(tail_out[0, 0, 2 * dk:, 2], v[1, 0])
    np.testing.assert_array_equal(tail_out[1], tail[1])
    np.testing.assert_array_equal(tail_out[2, 0, dk:2 * dk, :], raw[1][4:7, 0].T)
