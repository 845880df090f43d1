"""Plain fp64 CPU oracle for the KDA gated delta-rule recurrence.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import, call or link anything under ``oracle/``. The library's
product path never routes through this file, and this file imports nothing from it.

Everything here is written to be checked by eye against the pages, not to be fast:
per-token loops, fp64 arithmetic, inputs upcast exactly from the device bits.

Sources (page title, section):
* "Noyaux KDA et FlashKDA", section "Le conflit fondamental": each head carries a fixed
  state S of shape d_k x d_v that is updated serially, token by token.
* same page, section "Le rôle de la décroissance bornée": the per-key-channel log-decay is
  floored at g_min = -5.
* same page, section "FlashKDA : le noyau par blocs": the blockwise (chunk) form is parallel
  inside a chunk and serial across chunks.
* same page, section "Le parallélisme de contexte intra-appareil": a segment's state
  transition can be evaluated without its incoming state and composed exactly afterwards.
* AMD blog "Dentro de los esfuerzos de optimización de Kimi K3", section 5 (KDA: paralelizar
  el prellenado...): worked example of composing "halve and add two" with "halve and add
  one"; ordered scan of group summaries, then parallel replay.
* same blog, "Nota técnica: Precisión del KDA y memoria on-chip": the chunk's dependencies
  are folded into one transformation (the inverse of a unit lower-triangular dependency
  matrix); worked coefficient example with entries -1/4 and -1/16.
* "Noyaux d'inférence", section "1. Le décodage KDA": speculative verify replays the cached
  projected inputs of accepted draft tokens instead of snapshotting S; one fused loop covers
  short convolution, input normalisation, gating, the recurrence and output normalisation.

Readings where the pages are silent (each listed in the design doc):
* The update order is "decay, then delta correction, then read-out":
      S' = diag(exp(max(g_t, g_min))) S
      S  = S' + beta_t k_t (v_t - S'^T k_t)^T
      o_t = scale * S^T q_t
  The pages never print the update. The pins below check that this oracle implements that
  reading; no value printed on the pages tells the two possible update orders apart
  (parity of the ORDER itself is unpinned).
* Decode: depthwise causal convolution of width W over the raw q, k and v channels with a
  tail of the last W-1 raw inputs; SiLU after the convolution (flag ``act``); L2
  normalisation of q and k over d_k with eps inside the square root; beta = sigmoid(raw);
  g = max(-softplus(raw), g_min); gated RMSNorm of the output over d_v:
  o * rsqrt(mean(o^2) + eps) * w * sigmoid(z). These forms are readings: the pages name the
  steps but print none of their formulas (parity of those forms is unpinned beyond the
  special cases tested).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "recurrence_fwd",
    "recurrence_bwd",
    "token_transition",
    "brute_force_fwd",
    "chunk_log_decay",
    "chunk_dependency_matrix",
    "unit_lower_inverse",
    "chunked_fwd",
    "segment_transition",
    "segment_scan",
    "silu",
    "sigmoid",
    "softplus",
    "causal_conv_window",
    "decode_token",
    "decode_replay",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _seq_bounds(T, cu_seqlens):
    if cu_seqlens is None:
        return [(0, T)]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


# ---------------------------------------------------------------------------------------------
# Definition: per-token recurrence ("Noyaux KDA et FlashKDA", "Le conflit fondamental";
# floor from "Le rôle de la décroissance bornée").
# ---------------------------------------------------------------------------------------------
def recurrence_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=1.0, g_min=-5.0):
    """Run the KDA recurrence token by token.

    Shapes (packed varlen, B = 1): q, k, g: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H];
    h0: [N, H, d_k, d_v] or None (zeros); cu_seqlens: [N + 1] or None (one sequence).
    Returns (o [T, H, d_v], ht [N, H, d_k, d_v]) in fp64. A sequence of length 0 returns its
    h0 unchanged. Rows of S are key channels, columns value channels.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, H, dk = k.shape
    dv = v.shape[-1]
    bounds = _seq_bounds(T, cu_seqlens)
    o = np.zeros((T, H, dv))
    ht = np.zeros((len(bounds), H, dk, dv))
    for n, (bos, eos) in enumerate(bounds):
        S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0)[n].copy()
        for t in range(bos, eos):
            a = np.exp(np.maximum(g[t], g_min))                 # [H, d_k] per-channel decay
            S = a[:, :, None] * S                               # decay the key rows
            err = v[t] - np.einsum("hkv,hk->hv", S, k[t])       # delta error v - S'^T k
            S = S + beta[t][:, None, None] * k[t][:, :, None] * err[:, None, :]
            o[t] = scale * np.einsum("hkv,hk->hv", S, q[t])     # read-out after the update
        ht[n] = S
    return o, ht


def recurrence_bwd(q, k, v, g, beta, do, dht=None, h0=None, cu_seqlens=None, scale=1.0,
                   g_min=-5.0):
    """Gradients of recurrence_fwd by reverse-mode differentiation of the same per-token
    update (the pages give no backward: this is the chain rule applied to the forward
    definition above, one step at a time, in reverse token order).

    For a loss L with dL/do = ``do`` [T, H, d_v] and dL/dht = ``dht`` [N, H, d_k, d_v] (None:
    zeros), returns a dict of dq, dk, dg [T, H, d_k], dv [T, H, d_v], dbeta [T, H] and dh0
    [N, H, d_k, d_v], all fp64. Per token, with a = exp(max(g_t, g_min)):
        S' = diag(a) S_prev;  u = v_t - S'^T k_t;  S = S' + beta_t k_t u^T;  o_t = scale S^T q_t
    and, going backwards with D = dL/dS (starting from dht):
        D += scale q_t do_t^T;               dq_t = scale S do_t
        dbeta_t = k_t^T D u;                 du = beta_t D^T k_t;    dv_t = du
        D' = D - k_t du^T;                   dk_t = beta_t D u - S' du
        dg_t = a * rowsum(S_prev * D') where g_t > g_min, else 0 (the floor is flat)
        D = diag(a) D'                       (dL/dS_prev; dh0 is D at the sequence start)
    """
    q, k, v, g, beta, do = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta), _f64(do)
    T, H, dk = k.shape
    dv = v.shape[-1]
    bounds = _seq_bounds(T, cu_seqlens)
    grads = {"dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
             "dg": np.zeros((T, H, dk)), "dbeta": np.zeros((T, H)),
             "dh0": np.zeros((len(bounds), H, dk, dv))}
    for n, (bos, eos) in enumerate(bounds):
        # forward again, keeping what the reverse steps read
        S = np.zeros((H, dk, dv)) if h0 is None else _f64(h0)[n].copy()
        saved = []
        for t in range(bos, eos):
            a = np.exp(np.maximum(g[t], g_min))
            S_prev = S
            Sp = a[:, :, None] * S_prev
            u = v[t] - np.einsum("hkv,hk->hv", Sp, k[t])
            S = Sp + beta[t][:, None, None] * k[t][:, :, None] * u[:, None, :]
            saved.append((a, S_prev, Sp, u, S))
        D = np.zeros((H, dk, dv)) if dht is None else _f64(dht)[n].copy()
        for t in range(eos - 1, bos - 1, -1):
            a, S_prev, Sp, u, S = saved[t - bos]
            D = D + scale * q[t][:, :, None] * do[t][:, None, :]
            grads["dq"][t] = scale * np.einsum("hkv,hv->hk", S, do[t])
            Du = np.einsum("hkv,hv->hk", D, u)                   # D u
            grads["dbeta"][t] = np.einsum("hk,hk->h", k[t], Du)
            du = beta[t][:, None] * np.einsum("hkv,hk->hv", D, k[t])
            grads["dv"][t] = du
            Dp = D - k[t][:, :, None] * du[:, None, :]
            grads["dk"][t] = beta[t][:, None] * Du - np.einsum("hkv,hv->hk", Sp, du)
            live = g[t] > g_min
            grads["dg"][t] = np.where(live, a * np.einsum("hkv,hkv->hk", S_prev, Dp), 0.0)
            D = a[:, :, None] * Dp
        grads["dh0"][n] = D
    return grads


def token_transition(k_t, g_t, beta_t, g_min=-5.0):
    """The token's affine map S -> A_t S + b_t written as the explicit d_k x d_k matrix
    A_t = (I - beta k k^T) diag(exp(max(g, g_min))) (single head). The additive part is
    beta k v^T and is formed by the callers."""
    k_t, g_t = _f64(k_t), _f64(g_t)
    dk = k_t.shape[0]
    D = np.diag(np.exp(np.maximum(g_t, g_min)))
    return (np.eye(dk) - float(beta_t) * np.outer(k_t, k_t)) @ D


def brute_force_fwd(q, k, v, g, beta, h0, scale=1.0, g_min=-5.0):
    """Independent expansion for tiny T (single head): every state is written as
    S_t = (A_t ... A_1) S_0 + sum_s (A_t ... A_{s+1}) beta_s k_s v_s^T, with the transition
    products formed explicitly (no running state). Returns (o [T, d_v], S_T)."""
    q, k, v, g, beta, h0 = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta), _f64(h0)
    T, dk = k.shape
    As = [token_transition(k[t], g[t], beta[t], g_min) for t in range(T)]
    o = np.zeros((T, v.shape[1]))
    S_t = h0
    for t in range(T):
        prod = np.eye(dk)
        for s in range(t + 1):
            prod = As[s] @ prod
        S_t = prod @ h0
        for s in range(t + 1):
            tail = np.eye(dk)
            for u in range(s + 1, t + 1):
                tail = As[u] @ tail
            S_t = S_t + tail @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = scale * S_t.T @ q[t]
    return o, S_t


# ---------------------------------------------------------------------------------------------
# Second formulation: the chunk (UT/WY) form. Used only to cross-check the definition and the
# worked coefficient example ("Nota técnica: Precisión del KDA y memoria on-chip";
# "FlashKDA : le noyau par blocs").
# ---------------------------------------------------------------------------------------------
def chunk_log_decay(g, g_min=-5.0):
    """In-chunk cumulative log-decay Gamma_r = sum_{s<=r} max(g_s, g_min) per key channel."""
    return np.cumsum(np.maximum(_f64(g), g_min), axis=0)


def chunk_dependency_matrix(k, g, beta, g_min=-5.0):
    """Strictly lower-triangular A with A[r, s] = beta_r * sum_i k[r,i] k[s,i]
    exp(Gamma[r,i] - Gamma[s,i]) for s < r: how token s's correction feeds token r's error
    inside one chunk (single head, k: [L, d_k])."""
    k, beta = _f64(k), _f64(beta)
    gam = chunk_log_decay(g, g_min)
    L = k.shape[0]
    A = np.zeros((L, L))
    for r in range(L):
        for s in range(r):
            A[r, s] = beta[r] * np.sum(k[r] * k[s] * np.exp(gam[r] - gam[s]))
    return A


def unit_lower_inverse(A):
    """(I + A)^{-1} for strictly lower-triangular A by forward substitution: entry (r, s)
    sums every dependency path from position s to position r."""
    A = _f64(A)
    L = A.shape[0]
    T = np.eye(L)
    for r in range(L):
        for s in range(r):
            T[r, s] = -np.dot(A[r, s:r], T[s:r, s])
    return T


def chunked_fwd(q, k, v, g, beta, h0=None, scale=1.0, g_min=-5.0, chunk=64):
    """Chunk form of recurrence_fwd for one sequence (q, k, g: [T, H, d_k]).

    Per chunk with entering state S: Gamma = cumsum(max(g, g_min)); Tm = (I + A)^{-1};
    W = Tm diag(beta) (K * e^Gamma); U = Tm diag(beta) V - W S;
    M[r, s] = sum_i q[r,i] k[s,i] e^{Gamma[r,i]-Gamma[s,i]} for s <= r;
    O = scale (Q * e^Gamma) S + scale M U;  S <- diag(e^{Gamma_L}) S + (K * e^{Gamma_L - Gamma})^T U.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((T, H, dv))
    ht = np.zeros((H, dk, dv))
    for h in range(H):
        S = np.zeros((dk, dv)) if h0 is None else _f64(h0)[h].copy()
        for c0 in range(0, T, chunk):
            c1 = min(c0 + chunk, T)
            qc, kc, vc, gc, bc = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h], beta[c0:c1, h]
            gam = chunk_log_decay(gc, g_min)
            Tm = unit_lower_inverse(chunk_dependency_matrix(kc, gc, bc, g_min))
            W = Tm @ (bc[:, None] * (kc * np.exp(gam)))
            U = Tm @ (bc[:, None] * vc) - W @ S
            L = c1 - c0
            M = np.zeros((L, L))
            for r in range(L):
                for s in range(r + 1):
                    M[r, s] = np.sum(qc[r] * kc[s] * np.exp(gam[r] - gam[s]))
            o[c0:c1, h] = scale * ((qc * np.exp(gam)) @ S + M @ U)
            S = np.exp(gam[-1])[:, None] * S + (kc * np.exp(gam[-1] - gam)).T @ U
        ht[h] = S
    return o, ht


# ---------------------------------------------------------------------------------------------
# Segment transitions and the ordered scan ("Le parallélisme de contexte intra-appareil";
# AMD blog section 5).
# ---------------------------------------------------------------------------------------------
def segment_transition(k, v, g, beta, g_min=-5.0):
    """Affine summary (P, Q) of a segment for one head, built without its incoming state:
    S_out = P S_in + Q. Composes the per-token maps S -> A_t S + beta_t k_t v_t^T in order."""
    k, v, beta = _f64(k), _f64(v), _f64(beta)
    dk, dv = k.shape[1], v.shape[1]
    P = np.eye(dk)
    Q = np.zeros((dk, dv))
    for t in range(k.shape[0]):
        A_t = token_transition(k[t], g[t], beta[t], g_min)
        P = A_t @ P
        Q = A_t @ Q + beta[t] * np.outer(k[t], v[t])
    return P, Q


def segment_scan(h0, Ps, Qs):
    """Ordered scan: S_in(0) = h0, S_in(j+1) = P_j S_in(j) + Q_j. Returns the list of every
    segment's entering state plus the final state (length n_seg + 1)."""
    S = _f64(h0).copy()
    states = [S]
    for P, Q in zip(Ps, Qs):
        S = _f64(P) @ S + _f64(Q)
        states.append(S)
    return states


# ---------------------------------------------------------------------------------------------
# Decode: fused speculative-verify replay ("Noyaux d'inférence", "1. Le décodage KDA";
# AMD blog section 3 for the single-token fused path).
# ---------------------------------------------------------------------------------------------
def silu(x):
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def sigmoid(x):
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    return np.logaddexp(0.0, _f64(x))


def causal_conv_window(tail, x, w):
    """One step of a depthwise causal convolution for each channel.

    tail: [C, W-1] previous raw inputs, oldest first; x: [C] current raw input; w: [C, W]
    taps, w[:, W-1] multiplies the current input. Returns (y [C], new tail [C, W-1])."""
    win = np.concatenate([_f64(tail), _f64(x)[:, None]], axis=1)
    return np.sum(win * _f64(w), axis=1), win[:, 1:]


def decode_token(S, tail, x, conv_w, norm_w, scale, g_min, eps_l2, eps_rms, act, output):
    """One decode token for one (request, head).

    S: [d_k, d_v]; tail: [2 d_k + d_v, W-1] (channel order q, k, v); x: dict with raw 'q',
    'k' [d_k], 'v' [d_v], 'g' [d_k], 'beta' scalar and, when ``output``, 'z' [d_v];
    conv_w: [2 d_k + d_v, W]. Returns (S, tail, o or None)."""
    dk, dv = S.shape
    raw = np.concatenate([_f64(x["q"]), _f64(x["k"]), _f64(x["v"])])
    y, tail = causal_conv_window(tail, raw, conv_w)
    if act:
        y = silu(y)
    q, k, v = y[:dk], y[dk:2 * dk], y[2 * dk:]
    q = q / np.sqrt(np.sum(q * q) + eps_l2)
    k = k / np.sqrt(np.sum(k * k) + eps_l2)
    beta = float(sigmoid(x["beta"]))
    g = np.maximum(-softplus(x["g"]), g_min)
    S = np.exp(g)[:, None] * S
    S = S + beta * np.outer(k, v - S.T @ k)
    if not output:
        return S, tail, None
    o = scale * (S.T @ q)
    o = o / np.sqrt(np.mean(o * o) + eps_rms) * _f64(norm_w) * sigmoid(x["z"])
    return S, tail, o


def _window_token(win, r, j, h):
    tok = {name: win[name][r, j, h] for name in ("q", "k", "v", "g", "beta")}
    if "z" in win and win["z"] is not None:
        tok["z"] = win["z"][r, j, h]
    return tok


def decode_replay(state, conv_tail, n_acc, prev, new, conv_w, norm_w, scale=1.0, g_min=-5.0,
                  eps_l2=1e-6, eps_rms=1e-6, act=1):
    """Speculative-verify step for R requests and H heads.

    state: [R, H, d_k, d_v] committed state (after the previous bonus token);
    conv_tail: [R, H, 2 d_k + d_v, W-1]; n_acc: [R] accepted drafts of the previous window;
    prev / new: dicts of raw projected inputs, each tensor [R, slots, H, ...] ('beta'
    [R, slots, H]); prev slot 0 is the previous bonus (already committed), slots 1..n_acc are
    the accepted drafts replayed here; new slot 0 is the bonus token, slots 1.. the next
    draft window. conv_w: [H, 2 d_k + d_v, W]; norm_w: [d_v].

    Returns dict(o [R, n_new, H, d_v], state (after the bonus, the new committed state),
    state_acc (after the replayed drafts), conv_tail (after the bonus)).
    """
    state, conv_tail = _f64(state), _f64(conv_tail)
    R, H, dk, dv = state.shape
    n_new = new["q"].shape[1]
    o = np.zeros((R, n_new, H, dv))
    out_state = np.zeros_like(state)
    out_acc = np.zeros_like(state)
    out_tail = np.zeros_like(conv_tail)
    for r in range(R):
        for h in range(H):
            S, tail = state[r, h].copy(), conv_tail[r, h].copy()
            args = (conv_w[h], norm_w, scale, g_min, eps_l2, eps_rms, act)
            for j in range(1, int(n_acc[r]) + 1):
                S, tail, _ = decode_token(S, tail, _window_token(prev, r, j, h), *args, output=False)
            out_acc[r, h] = S
            for j in range(n_new):
                S, tail, o[r, j, h] = decode_token(S, tail, _window_token(new, r, j, h), *args,
                                                   output=True)
                if j == 0:
                    out_state[r, h] = S
                    out_tail[r, h] = tail
    return {"o": o, "state": out_state, "state_acc": out_acc, "conv_tail": out_tail}


# ---------------------------------------------------------------------------------------------
# Prefill from raw projections: the decode's token stage (short convolution, SiLU, L2 input
# norms, gate activations; "Noyaux d'inférence", section "1. Le décodage KDA") applied to every
# token of a sequence in order, then the recurrence.
# ---------------------------------------------------------------------------------------------
def prefill_input_stage(q_raw, k_raw, v_raw, g_raw, beta_raw, conv_w, conv_tail=None,
                        cu_seqlens=None, act=1, eps_l2=1e-6, g_min=-5.0):
    """Token stage of every token, sequence by sequence and in token order.

    q_raw, k_raw, g_raw: [T, H, d_k]; v_raw: [T, H, d_v]; beta_raw: [T, H]; conv_w:
    [H, 2 d_k + d_v, W]; conv_tail: [N, H, 2 d_k + d_v, W-1] raw inputs before each sequence
    (zeros if None). Returns (q, k, v, g, beta, conv_tail_out) with the tail after each
    sequence's last token."""
    q_raw, k_raw, v_raw = _f64(q_raw), _f64(k_raw), _f64(v_raw)
    g_raw, beta_raw, conv_w = _f64(g_raw), _f64(beta_raw), _f64(conv_w)
    T, H, dk = q_raw.shape
    dv = v_raw.shape[-1]
    W = conv_w.shape[-1]
    bounds = _seq_bounds(T, cu_seqlens)
    q, k, v = np.zeros((T, H, dk)), np.zeros((T, H, dk)), np.zeros((T, H, dv))
    tail_out = np.zeros((len(bounds), H, 2 * dk + dv, W - 1))
    for n, (bos, eos) in enumerate(bounds):
        for h in range(H):
            tail = (np.zeros((2 * dk + dv, W - 1)) if conv_tail is None
                    else _f64(conv_tail)[n, h].copy())
            for t in range(bos, eos):
                raw = np.concatenate([q_raw[t, h], k_raw[t, h], v_raw[t, h]])
                y, tail = causal_conv_window(tail, raw, conv_w[h])
                if act:
                    y = silu(y)
                qq, kk = y[:dk], y[dk:2 * dk]
                q[t, h] = qq / np.sqrt(np.sum(qq * qq) + eps_l2)
                k[t, h] = kk / np.sqrt(np.sum(kk * kk) + eps_l2)
                v[t, h] = y[2 * dk:]
            tail_out[n, h] = tail
    beta = sigmoid(beta_raw)
    g = np.maximum(-softplus(g_raw), g_min)
    return q, k, v, g, beta, tail_out


def prefill_raw_fwd(q_raw, k_raw, v_raw, g_raw, beta_raw, conv_w, conv_tail=None, h0=None,
                    cu_seqlens=None, scale=1.0, g_min=-5.0, eps_l2=1e-6, act=1):
    """The raw prefill: the token stage above, then the recurrence. Returns (o, ht,
    conv_tail_out)."""
    q, k, v, g, beta, tail = prefill_input_stage(q_raw, k_raw, v_raw, g_raw, beta_raw, conv_w,
                                                 conv_tail, cu_seqlens, act, eps_l2, g_min)
    o, ht = recurrence_fwd(q, k, v, g, beta, h0=h0, cu_seqlens=cu_seqlens, scale=scale,
                           g_min=g_min)
    return o, ht, tail
