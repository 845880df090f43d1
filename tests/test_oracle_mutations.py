"""Mutation check of the oracle's pins (CPU).

Each case plants one plausible mistake in the oracle (a dropped term, a wrong sign, an
index off by one, a swapped operand or order) by replacing one of its functions for the
duration of the test, then runs the pins of test_oracle_pins.py and requires at least one
of them to fail. The comparison with the C twin is left out: it would flag any change of
the NumPy code and says nothing about the pages. So a passing case shows the pins, which
are all anchored outside the oracle (printed values, closed forms, brute force, invariants,
library routines), constrain that part of the oracle.
"""
import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import kda_oracle as ko

PINS = [
    ("worked example: segment composition", pins.test_worked_example_segment_composition, ()),
    ("worked example: dependency inverse", pins.test_worked_example_dependency_inverse, ()),
    ("closed form: beta = 0 with the floor", pins.test_closed_form_beta_zero_with_floor, ()),
    ("closed form: overwrite", pins.test_closed_form_overwrite_orthonormal_keys, ()),
    ("brute force", pins.test_brute_force_small, ()),
    ("chunked = per token", pins.test_chunked_equals_per_token, (150, 64)),
    ("chunked, floor stress", pins.test_chunked_with_floor_stress, ()),
    ("segment composition", pins.test_segment_composition_equals_full_run, ([0, 40, 90],)),
    ("linearity", pins.test_linearity_in_state_and_values, ()),
    ("heads and columns independent", pins.test_heads_and_value_columns_independent, ()),
    ("varlen and empty sequence", pins.test_varlen_packing_equals_separate_runs_and_empty_sequence, ()),
    ("contraction", pins.test_token_transition_is_a_contraction, ()),
    ("state energy bound", pins.test_state_column_energy_bound, ()),
    ("decode elementary functions", pins.test_decode_elementary_functions, ()),
    ("conv = np.convolve", pins.test_causal_conv_matches_numpy_convolve, ()),
    ("decode single token", pins.test_decode_single_token_is_one_recurrence_step, ()),
    ("decode stream lossless", pins.test_decode_speculative_stream_is_lossless, ()),
    ("decode output norm", pins.test_decode_output_norm_unit_rms, ()),
    ("raw prefill = decode token steps", pins.test_raw_prefill_matches_decode_token_steps, ()),
    ("raw prefill tails", pins.test_raw_prefill_tail_of_short_sequences, ()),
]


def failing_pins():
    failed = []
    for name, fn, args in PINS:
        try:
            with np.errstate(all="ignore"):
                fn(*args)
        except AssertionError:
            failed.append(name)
        except (ValueError, FloatingPointError, ZeroDivisionError, IndexError) as e:
            failed.append(f"{name} ({type(e).__name__})")
    return failed


# ------------------------------------------------------------------ mutants of the definition
def _recurrence(variant):
    """The per-token recurrence with one planted mistake."""
    def f(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=1.0, g_min=-5.0):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        T, H, dk = k.shape
        dv = v.shape[-1]
        bounds = ko._seq_bounds(T, cu_seqlens)
        o = np.zeros((T, H, dv))
        ht = np.zeros((len(bounds), H, dk, dv))
        for n, (bos, eos) in enumerate(bounds):
            S = np.zeros((H, dk, dv))
            if h0 is not None and variant != "h0 ignored":
                S = np.asarray(h0, dtype=np.float64)[n].copy()
            for t in range(bos, eos):
                gt = g[t]
                if variant == "floor missing":
                    a = np.exp(gt)
                elif variant == "floor as an upper clamp":
                    a = np.exp(np.minimum(gt, g_min))
                elif variant == "decay missing":
                    a = np.ones_like(gt)
                else:
                    a = np.exp(np.maximum(gt, g_min))
                b = np.ones_like(beta[t]) if variant == "beta missing" else beta[t]
                kt = k[t - 1] if (variant == "previous key in the error" and t > bos) else k[t]
                if variant != "correct, then decay":
                    S = a[:, :, None] * S
                pred = np.einsum("hkv,hk->hv", S, kt)
                err = v[t] + pred if variant == "delta sign" else v[t] - pred
                if variant == "read-out before the update":
                    o[t] = scale * np.einsum("hkv,hk->hv", S, q[t])
                S = S + b[:, None, None] * k[t][:, :, None] * err[:, None, :]
                if variant == "correct, then decay":
                    S = a[:, :, None] * S
                if variant != "read-out before the update":
                    sc = 1.0 if variant == "scale missing" else scale
                    o[t] = sc * np.einsum("hkv,hk->hv", S, q[t])
            ht[n] = S
        return o, ht
    return f


DEFINITION_MUTANTS = ["floor missing", "floor as an upper clamp", "decay missing",
                      "beta missing", "previous key in the error", "correct, then decay",
                      "delta sign", "read-out before the update", "h0 ignored",
                      "scale missing"]


@pytest.mark.parametrize("variant", DEFINITION_MUTANTS)
def test_definition_mutant_is_caught(variant, monkeypatch):
    monkeypatch.setattr(ko, "recurrence_fwd", _recurrence(variant))
    failed = failing_pins()
    print(f"{variant}: caught by {failed}")
    assert failed, f"no pin catches the mutant '{variant}'"


# ------------------------------------------------------------------ mutants of the other parts
def _token_transition(variant):
    def f(k_t, g_t, beta_t, g_min=-5.0):
        k_t, g_t = np.asarray(k_t, np.float64), np.asarray(g_t, np.float64)
        dk = k_t.shape[0]
        D = np.diag(np.exp(np.maximum(g_t, g_min)))
        R = np.eye(dk) - float(beta_t) * np.outer(k_t, k_t)
        if variant == "decay after the correction":
            return D @ R
        if variant == "correction sign":
            return (np.eye(dk) + float(beta_t) * np.outer(k_t, k_t)) @ D
        return R   # "decay missing"
    return f


def _unit_lower_inverse(variant):
    def f(A):
        A = np.asarray(A, np.float64)
        L = A.shape[0]
        T = np.eye(L)
        for r in range(L):
            for s in range(r):
                if variant == "inverse sign":
                    T[r, s] = np.dot(A[r, s:r], T[s:r, s])
                else:  # "inverse path sum short by one"
                    T[r, s] = -np.dot(A[r, s:r - 1], T[s:r - 1, s]) if r - 1 > s else -A[r, s]
        return T
    return f


def _chunk_log_decay(g, g_min=-5.0):
    """Exclusive instead of inclusive cumulative decay."""
    x = np.maximum(np.asarray(g, np.float64), g_min)
    return np.cumsum(x, axis=0) - x


def _dependency_swapped(k, g, beta, g_min=-5.0):
    """Decay exponent with rows and columns swapped."""
    k, beta = np.asarray(k, np.float64), np.asarray(beta, np.float64)
    gam = ko.chunk_log_decay(g, g_min)
    L = k.shape[0]
    A = np.zeros((L, L))
    for r in range(L):
        for s in range(r):
            A[r, s] = beta[r] * np.sum(k[r] * k[s] * np.exp(gam[s] - gam[r]))
    return A


def _segment_transition_late_decay(k, v, g, beta, g_min=-5.0):
    """Adds the token's correction before applying its map."""
    k, v, beta = np.asarray(k, np.float64), np.asarray(v, np.float64), np.asarray(beta, np.float64)
    P, Q = np.eye(k.shape[1]), np.zeros((k.shape[1], v.shape[1]))
    for t in range(k.shape[0]):
        A_t = ko.token_transition(k[t], g[t], beta[t], g_min)
        P = A_t @ P
        Q = A_t @ (Q + beta[t] * np.outer(k[t], v[t]))
    return P, Q


def _segment_scan_reversed(h0, Ps, Qs):
    """Composes the segments in the wrong order."""
    S = np.asarray(h0, np.float64).copy()
    states = [S]
    for P, Q in zip(reversed(list(Ps)), reversed(list(Qs))):
        S = P @ S + Q
        states.append(S)
    return states


def _conv_newest_first(tail, x, w):
    win = np.concatenate([np.asarray(x, np.float64)[:, None], np.asarray(tail, np.float64)], 1)
    return np.sum(win * np.asarray(w, np.float64), axis=1), win[:, :-1]


def _decode_token(variant):
    def f(S, tail, x, conv_w, norm_w, scale, g_min, eps_l2, eps_rms, act, output):
        dk, dv = S.shape
        raw = np.concatenate([np.asarray(x["q"], np.float64), np.asarray(x["k"], np.float64),
                              np.asarray(x["v"], np.float64)])
        y, tail = ko.causal_conv_window(tail, raw, conv_w)
        if act and variant != "SiLU missing":
            y = ko.silu(y)
        q, k, v = y[:dk], y[dk:2 * dk], y[2 * dk:]
        q = q / np.sqrt(np.sum(q * q) + eps_l2)
        if variant != "key norm missing":
            k = k / np.sqrt(np.sum(k * k) + eps_l2)
        beta = float(x["beta"]) if variant == "beta gate missing" else float(ko.sigmoid(x["beta"]))
        g = np.maximum(-ko.softplus(x["g"]), g_min)
        if variant == "decay gate sign":
            g = np.maximum(ko.softplus(x["g"]) * -0.5, g_min)
        S = np.exp(g)[:, None] * S
        S = S + beta * np.outer(k, v - S.T @ k)
        if not output:
            return S, tail, None
        o = scale * (S.T @ q)
        gate = 1.0 if variant == "output gate missing" else ko.sigmoid(x["z"])
        w = 1.0 if variant == "norm weight missing" else np.asarray(norm_w, np.float64)
        o = o / np.sqrt(np.mean(o * o) + eps_rms) * w * gate
        return S, tail, o
    return f


def _prefill_stage(variant):
    """The raw prefill's token stage with one planted mistake."""
    def f(q_raw, k_raw, v_raw, g_raw, beta_raw, conv_w, conv_tail=None, cu_seqlens=None, act=1,
          eps_l2=1e-6, g_min=-5.0):
        q_raw, k_raw, v_raw = (np.asarray(x, np.float64) for x in (q_raw, k_raw, v_raw))
        conv_w = np.asarray(conv_w, np.float64)
        T, H, dk = q_raw.shape
        dv = v_raw.shape[-1]
        W = conv_w.shape[-1]
        bounds = ko._seq_bounds(T, cu_seqlens)
        q, k, v = np.zeros((T, H, dk)), np.zeros((T, H, dk)), np.zeros((T, H, dv))
        tail_out = np.zeros((len(bounds), H, 2 * dk + dv, W - 1))
        for n, (bos, eos) in enumerate(bounds):
            for h in range(H):
                start = (np.zeros((2 * dk + dv, W - 1)) if conv_tail is None
                         or variant == "entering tail ignored"
                         else np.asarray(conv_tail, np.float64)[n, h].copy())
                tail = start.copy()
                for t in range(bos, eos):
                    raw = np.concatenate([q_raw[t, h], k_raw[t, h], v_raw[t, h]])
                    y, new_tail = ko.causal_conv_window(tail, raw, conv_w[h])
                    if variant != "tail not carried":
                        tail = new_tail
                    if act:
                        y = ko.silu(y)
                    qq, kk = y[:dk], y[dk:2 * dk]
                    q[t, h] = qq / np.sqrt(np.sum(qq * qq) + eps_l2)
                    k[t, h] = kk if variant == "key norm missing" else kk / np.sqrt(np.sum(kk * kk) + eps_l2)
                    v[t, h] = v_raw[t, h] if variant == "value conv skipped" else y[2 * dk:]
                tail_out[n, h] = start if variant == "leaving tail not written" else tail
        beta = ko.sigmoid(beta_raw)
        g = np.maximum(-ko.softplus(g_raw), g_min)
        return q, k, v, g, beta, tail_out
    return f


OTHER_MUTANTS = {
    "token map: decay after the correction": ("token_transition", _token_transition("decay after the correction")),
    "token map: correction sign": ("token_transition", _token_transition("correction sign")),
    "token map: decay missing": ("token_transition", _token_transition("decay missing")),
    "inverse: sign": ("unit_lower_inverse", _unit_lower_inverse("inverse sign")),
    "inverse: path sum short by one": ("unit_lower_inverse", _unit_lower_inverse("short")),
    "chunk decay: exclusive cumsum": ("chunk_log_decay", _chunk_log_decay),
    "dependency matrix: exponent swapped": ("chunk_dependency_matrix", _dependency_swapped),
    "segment summary: correction before the map": ("segment_transition", _segment_transition_late_decay),
    "segment scan: reversed order": ("segment_scan", _segment_scan_reversed),
    "conv: window newest first": ("causal_conv_window", _conv_newest_first),
    "decode: SiLU missing": ("decode_token", _decode_token("SiLU missing")),
    "decode: key norm missing": ("decode_token", _decode_token("key norm missing")),
    "decode: beta gate missing": ("decode_token", _decode_token("beta gate missing")),
    "decode: decay gate wrong": ("decode_token", _decode_token("decay gate sign")),
    "decode: output gate missing": ("decode_token", _decode_token("output gate missing")),
    "decode: norm weight missing": ("decode_token", _decode_token("norm weight missing")),
    "raw prefill: key norm missing": ("prefill_input_stage", _prefill_stage("key norm missing")),
    "raw prefill: tail not carried": ("prefill_input_stage", _prefill_stage("tail not carried")),
    "raw prefill: entering tail ignored": ("prefill_input_stage", _prefill_stage("entering tail ignored")),
    "raw prefill: value conv skipped": ("prefill_input_stage", _prefill_stage("value conv skipped")),
    "raw prefill: leaving tail not written": ("prefill_input_stage", _prefill_stage("leaving tail not written")),
}


@pytest.mark.parametrize("name", sorted(OTHER_MUTANTS))
def test_other_mutant_is_caught(name, monkeypatch):
    attr, fn = OTHER_MUTANTS[name]
    monkeypatch.setattr(ko, attr, fn)
    failed = failing_pins()
    print(f"{name}: caught by {failed}")
    assert failed, f"no pin catches the mutant '{name}'"


# ------------------------------------------------------------------ mutants of the backward
import test_oracle_backward as bwd_pins  # noqa: E402

BACKWARD_PINS = [
    ("backward: central differences", bwd_pins.test_gradients_match_central_differences),
    ("backward: beta = 0 closed forms", bwd_pins.test_beta_zero_closed_forms),
    ("backward: floored decay", bwd_pins.test_floored_decay_gets_no_gradient),
]


def _backward(variant):
    """recurrence_bwd with one planted mistake."""
    def f(q, k, v, g, beta, do, dht=None, h0=None, cu_seqlens=None, scale=1.0, g_min=-5.0):
        q, k, v, g, beta, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta, do))
        T, H, dk = k.shape
        dv = v.shape[-1]
        cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
        out = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
               "dg": np.zeros((T, H, dk)), "dbeta": np.zeros((T, H)),
               "dh0": np.zeros((len(cu) - 1, H, dk, dv))}
        for n in range(len(cu) - 1):
            bos, eos = cu[n], cu[n + 1]
            S = np.zeros((H, dk, dv)) if h0 is None else np.asarray(h0, np.float64)[n].copy()
            saved = []
            for t in range(bos, eos):
                a = np.exp(np.maximum(g[t], g_min))
                Sp = a[:, :, None] * S
                u = v[t] - np.einsum("hkv,hk->hv", Sp, k[t])
                S_new = Sp + beta[t][:, None, None] * k[t][:, :, None] * u[:, None, :]
                saved.append((a, S, Sp, u, S_new))
                S = S_new
            D = np.zeros((H, dk, dv)) if dht is None else np.asarray(dht, np.float64)[n].copy()
            for t in range(eos - 1, bos - 1, -1):
                a, S_prev, Sp, u, S_t = saved[t - bos]
                if variant != "read-out term dropped":
                    D = D + scale * q[t][:, :, None] * do[t][:, None, :]
                S_read = Sp if variant == "dq from the state before the update" else S_t
                out["dq"][t] = scale * np.einsum("hkv,hv->hk", S_read, do[t])
                Du = np.einsum("hkv,hv->hk", D, u)
                out["dbeta"][t] = np.einsum("hk,hk->h", k[t], Du)
                du = beta[t][:, None] * np.einsum("hkv,hk->hv", D, k[t])
                out["dv"][t] = du
                Dp = D - k[t][:, :, None] * du[:, None, :]
                sgn = 1.0 if variant == "dk error-path sign" else -1.0
                out["dk"][t] = beta[t][:, None] * Du + sgn * np.einsum("hkv,hv->hk", Sp, du)
                live = np.ones_like(g[t], bool) if variant == "floor mask missing" else g[t] > g_min
                out["dg"][t] = np.where(live, a * np.einsum("hkv,hkv->hk", S_prev, Dp), 0.0)
                D = Dp if variant == "decay not carried back" else a[:, :, None] * Dp
            out["dh0"][n] = D
        return out
    return f


BACKWARD_MUTANTS = ["read-out term dropped", "dq from the state before the update",
                    "dk error-path sign", "floor mask missing", "decay not carried back"]


def test_backward_reimplementation_is_faithful(monkeypatch):
    """The unmutated reimplementation passes every backward pin (so a caught mutant is caught
    for its planted mistake)."""
    monkeypatch.setattr(ko, "recurrence_bwd", _backward("none"))
    for _, fn in BACKWARD_PINS:
        fn()


@pytest.mark.parametrize("variant", BACKWARD_MUTANTS)
def test_backward_mutant_is_caught(variant, monkeypatch):
    monkeypatch.setattr(ko, "recurrence_bwd", _backward(variant))
    failed = []
    for name, fn in BACKWARD_PINS:
        try:
            with np.errstate(all="ignore"):
                fn()
        except AssertionError:
            failed.append(name)
    assert failed, f"no backward pin caught the mutant '{variant}'"
