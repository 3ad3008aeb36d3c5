"""fp64 CPU oracle of the Gated DeltaNet layer -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
use this module.  The product path (the HIP library and its binding) never
imports it, and it imports nothing from the product path.

Sources.  The pages followed here are cited by title and section:

  [Hybrid]  "Hybrid transformers under load: where Gated DeltaNet loses to
            full attention" (braintools.ru).  Section 3 describes the layer in
            words: each token first decays the state through a learned gate,
            then overwrites what the state returns for the token's key with
            the token's value (the delta rule), instead of only adding to it;
            the introduction names the method's paper, Gated DeltaNet,
            arXiv:2412.06464.  Section 3 also states that the
            state has a fixed size whatever the context length; section 4.1
            prints the state byte counts; section 9 keeps states in fp32.
            Sections 3, 4.2 and 6.1 motivate state checkpoints at block
            boundaries for prefix reuse and measure their cost.
  [Forge]   "Forge: how I wrote my own inference engine and beat llama.cpp".
            Entry of 27 August: speculative verify of k draft rows, with
            state snapshots between rows so that rollback is a copy.
  [Strata]  "Chapter 6: engine startup and memory plan" (SSE Strata book),
            section 6.2: the GDN geometry (state size 128, 16 k-heads,
            48 v-heads, conv width 4, 10240 conv channels).

The rule written out (the gated delta rule of arXiv:2412.06464), per v-head
with state S of shape d_v x d_k:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = S_t q_t

with alpha_t = exp(g_t), g_t = -softplus(a_t), beta_t = sigmoid(b_t), and the
inputs q, k, v produced from the projected input x by a causal depthwise
conv of width W, SiLU, and an L2 normalisation of q and k.

Readings where the pages leave a step open (each is listed with its reason
in the design notes):
  * output scale: o_t = q_scale * S_t q_t with q_scale = 1 as the rule is written;
  * L2 normalisation: x * (sum x^2 + eps)^(-1/2), eps = 1e-6, per k-head over d_k,
    on q and k only, and only when the layer's conv front end is on;
  * channel order of the conv input: q | k | v, each head-major, dim-minor;
  * v-head h reads k-head floor(h / (H_v / H_k));
  * SiLU on all channels after the conv, no conv bias;
  * conv taps: w[c][W-1] multiplies the current token, w[c][0] the oldest;
  * softplus(x) = max(x, 0) + log1p(exp(-|x|)) with no threshold;
  * verify rows are exactly the k drafts; rollback(a) returns the state and the
    conv history after the first a drafts (a = 0: the state before verify).

Nothing here is blocked, fused or reordered beyond the rule: the sequential
functions loop over tokens and apply the rule one token at a time.  The
chunked form in ``chunked_recurrence`` exists only so that the tests can pin
the sequential form against an independent derivation.
"""
from __future__ import annotations

import numpy as np

try:  # scipy gives a library triangular solve for the chunked self-check
    from scipy.linalg import solve_triangular as _solve_tri
except Exception:  # pragma: no cover
    _solve_tri = None

F64 = np.float64


# ----------------------------------------------------------------------------
# Scalar laws: gates and activations ([Hybrid] section 3 names the gate; the
# exact laws are beta = sigmoid(b) and log alpha = -softplus(a)).
# ----------------------------------------------------------------------------

def softplus(x):
    """softplus(x) = log(1 + e^x), in the overflow-free form max(x,0) + log1p(e^-|x|)."""
    x = np.asarray(x, F64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow for either sign."""
    x = np.asarray(x, F64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(y):
    """SiLU(y) = y * sigmoid(y)."""
    y = np.asarray(y, F64)
    return y * sigmoid(y)


def gates(a, b):
    """Return (g, alpha, beta): g = -softplus(a) = log alpha, beta = sigmoid(b)."""
    g = -softplus(a)
    return g, np.exp(g), sigmoid(b)


def l2norm(x, eps):
    """x * (sum(x^2) + eps)^(-1/2) over the last axis."""
    x = np.asarray(x, F64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)


# ----------------------------------------------------------------------------
# Front end: causal depthwise conv of width W + SiLU, split, L2 norm.
# ----------------------------------------------------------------------------

def conv_silu(window, w):
    """One output row of the causal depthwise conv followed by SiLU.

    window: (W, C) inputs, oldest first, the last row being the current token.
    w:      (C, W) taps; w[c][W-1] multiplies the current token.
    Returns y (C,) with y[c] = SiLU(sum_j w[c][j] * window[j][c]).
    """
    window = np.asarray(window, F64)
    w = np.asarray(w, F64)
    y = np.einsum("cj,jc->c", w, window)
    return silu(y)


def split_qkv(y, geom):
    """Split a channel vector into q (H_k,d_k), k (H_k,d_k), v (H_v,d_v)."""
    nq = geom.n_k_heads * geom.d_k
    q = y[:nq].reshape(geom.n_k_heads, geom.d_k)
    k = y[nq:2 * nq].reshape(geom.n_k_heads, geom.d_k)
    v = y[2 * nq:].reshape(geom.n_v_heads, geom.d_v)
    return q, k, v


def frontend(window, w, geom):
    """q, k, v of one token from its conv window (or from x itself when W = 0).

    With the conv switched off (conv_width = 0) the input row already holds
    q | k | v and nothing is applied to it.
    """
    if geom.conv_width == 0:
        y = np.asarray(window[-1], F64)
    else:
        y = conv_silu(window, w)
    q, k, v = split_qkv(y, geom)
    if geom.l2norm_qk and geom.conv_width > 0:
        q = l2norm(q, geom.l2_eps)
        k = l2norm(k, geom.l2_eps)
    return q, k, v


def expand_heads(qk, geom):
    """Map k-head vectors (H_k, d_k) to the v-heads that read them (H_v, d_k)."""
    return np.repeat(qk, geom.group, axis=0)


# ----------------------------------------------------------------------------
# The gated delta rule, one token.
# ----------------------------------------------------------------------------

def delta_rule_step(S, q, k, v, g, beta, q_scale=1.0):
    """One token of the gated delta rule for every v-head at once.

    S (H,d_v,d_k), q and k (H,d_k), v (H,d_v), g and beta (H,).
    S_t = alpha S (I - beta k k^T) + beta v k^T, expanded without forming the
    d_k x d_k matrix: alpha S (I - beta k k^T) = alpha S - beta (alpha S k) k^T.
    Returns (S_t, o_t) with o_t = q_scale * S_t q_t.
    """
    alpha = np.exp(np.asarray(g, F64))
    beta = np.asarray(beta, F64)
    Sa = alpha[:, None, None] * S
    Sak = np.einsum("hij,hj->hi", Sa, k)
    S_new = Sa - beta[:, None, None] * Sak[:, :, None] * k[:, None, :] \
        + beta[:, None, None] * v[:, :, None] * k[:, None, :]
    o = q_scale * np.einsum("hij,hj->hi", S_new, q)
    return S_new, o


def delta_rule_step_matrix(S, q, k, v, g, beta, q_scale=1.0):
    """The same step with the transition matrix (I - beta k k^T) formed explicitly.

    The rule exactly as it is written, for small d: the pins compare the
    expanded form above with it, and check both against the transition's
    closed-form action on k and on the directions orthogonal to k.
    """
    H, dv, dk = S.shape
    out_S = np.empty_like(S, dtype=F64)
    out_o = np.empty((H, dv), F64)
    for h in range(H):
        M = np.eye(dk) - beta[h] * np.outer(k[h], k[h])
        out_S[h] = np.exp(g[h]) * (S[h] @ M) + beta[h] * np.outer(v[h], k[h])
        out_o[h] = q_scale * (out_S[h] @ q[h])
    return out_S, out_o


def recurrence(q, k, v, g, beta, S0, q_scale=1.0):
    """Sequential gated delta rule over T tokens (inputs already per v-head).

    q, k (T,H,d_k); v (T,H,d_v); g, beta (T,H); S0 (H,d_v,d_k).
    Returns (o (T,H,d_v), S_T).
    """
    S = np.array(S0, F64)
    T = q.shape[0]
    o = np.empty((T,) + v.shape[1:], F64)
    for t in range(T):
        S, o[t] = delta_rule_step(S, q[t], k[t], v[t], g[t], beta[t], q_scale)
    return o, S


# ----------------------------------------------------------------------------
# The layer over one sequence (conv history -> outputs, final state, history).
# ----------------------------------------------------------------------------

def layer_sequence(geom, x, a, b, conv_w, S0, hist0, heads=None):
    """Run the layer over one sequence, token by token.

    x (T,C); a, b (T,H_v); conv_w (C,W); S0 (H_v,d_v,d_k); hist0 (W-1,C) oldest
    first.  ``heads`` optionally restricts the recurrence to a list of v-heads
    (heads do not interact after the front end; the front end is still run on
    every channel).  Returns (o (T,H,d_v), S_T (H,d_v,d_k), hist_T (W-1,C)).
    """
    x = np.asarray(x, F64)
    T = x.shape[0]
    W = geom.conv_width
    heads = np.arange(geom.n_v_heads) if heads is None else np.asarray(heads)
    hist = np.asarray(hist0, F64).reshape(max(W - 1, 0), geom.conv_channels)
    S = np.array(np.asarray(S0, F64)[heads])
    g_all, _, beta_all = gates(a, b)
    o = np.empty((T, len(heads), geom.d_v), F64)
    for t in range(T):
        window = np.concatenate([hist, x[t:t + 1]], axis=0)
        q, k, v = frontend(window, conv_w, geom)
        qh = expand_heads(q, geom)[heads]
        kh = expand_heads(k, geom)[heads]
        S, o[t] = delta_rule_step(S, qh, kh, v[heads], g_all[t][heads],
                                  beta_all[t][heads], geom.q_scale)
        if W > 1:
            hist = window[1:]
    return o, S, hist


def decode_step(geom, state, hist, x, a, b, conv_w, slots):
    """One decode token per batch row on a slot pool.

    state (n_slots,H_v,d_v,d_k) and hist (n_slots,W-1,C) are the pool; x (B,C),
    a, b (B,H_v); slots (B,).  Returns (o (B,H_v,d_v), new_state, new_hist):
    slots not named in ``slots`` are returned unchanged.
    """
    state = np.array(state, F64)
    hist = np.array(hist, F64)
    o = np.empty((len(slots), geom.n_v_heads, geom.d_v), F64)
    for i, s in enumerate(slots):
        oi, state[s], hist[s] = layer_sequence(geom, x[i:i + 1], a[i:i + 1], b[i:i + 1],
                                               conv_w, state[s], hist[s])
        o[i] = oi[0]
    return o, state, hist


def verify(geom, S0, hist0, x, a, b, conv_w, heads=None):
    """Speculative verify of k drafts on one slot ([Forge], 27 August).

    Runs the rule over the k draft tokens and keeps the state and conv history
    after every draft.  The committed state is not modified.
    Returns (o (k,H,d_v), snaps (k,H,d_v,d_k), hists (k,W-1,C)).
    """
    kdr = x.shape[0]
    heads = np.arange(geom.n_v_heads) if heads is None else np.asarray(heads)
    S = np.array(np.asarray(S0, F64))
    hist = np.array(hist0, F64)
    o = np.empty((kdr, len(heads), geom.d_v), F64)
    snaps = np.empty((kdr, len(heads), geom.d_v, geom.d_k), F64)
    hists = np.empty((kdr,) + hist.shape, F64)
    for j in range(kdr):
        oj, S, hist = layer_sequence(geom, x[j:j + 1], a[j:j + 1], b[j:j + 1], conv_w,
                                     S, hist, heads=heads)
        S_full = S
        o[j] = oj[0]
        snaps[j] = S_full
        hists[j] = hist
        # keep S indexed by the selected heads for the next draft
        S = np.zeros((geom.n_v_heads, geom.d_v, geom.d_k), F64)
        S[heads] = S_full
    return o, snaps, hists


def rollback(S0, hist0, snaps, hists, accepted):
    """State and conv history after ``accepted`` drafts (0 returns the inputs)."""
    if accepted == 0:
        return np.array(S0, F64), np.array(hist0, F64)
    return np.array(snaps[accepted - 1]), np.array(hists[accepted - 1])


def prefill(geom, x, a, b, conv_w, cu_seqlens, S0s, hist0s, has_init, heads=None):
    """Variable-length prefill: each sequence [cu[s], cu[s+1]) runs on its own.

    S0s (S,H_v,d_v,d_k) and hist0s (S,W-1,C) are the initial states of the
    sequences, used only where has_init[s] is nonzero (zero otherwise).
    Returns (o (N,H,d_v), finals list of (S_T, hist_T)).
    """
    N = x.shape[0]
    heads = np.arange(geom.n_v_heads) if heads is None else np.asarray(heads)
    o = np.empty((N, len(heads), geom.d_v), F64)
    finals = []
    for s in range(len(cu_seqlens) - 1):
        t0, t1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        if has_init[s]:
            S0, h0 = np.asarray(S0s[s], F64), np.asarray(hist0s[s], F64)
        else:
            S0 = np.zeros((geom.n_v_heads, geom.d_v, geom.d_k), F64)
            h0 = np.zeros((max(geom.conv_width - 1, 0), geom.conv_channels), F64)
        o[t0:t1], S_T, h_T = layer_sequence(geom, x[t0:t1], a[t0:t1], b[t0:t1], conv_w,
                                            S0, h0, heads=heads)
        finals.append((S_T, h_T))
    return o, finals


def prefill_checkpoints(geom, x, a, b, conv_w, cu_seqlens, S0s, hist0s, has_init, every,
                        heads=None):
    """Variable-length prefill that also keeps the state at block boundaries.

    [Hybrid] section 3: a later request can reuse a shared prefix only through
    a copy of the state saved where the prefix ends, since the live state goes
    on to absorb the first request's own tail; section 4.2: such snapshots are
    taken at every cache-block boundary, and section 6.1 measures what writing
    them costs the prefill.  Here checkpoint j of sequence s is the state after
    the first (j+1)*every tokens of s, for every (j+1)*every <= len(s): the
    final state of the layer run over those tokens alone.  Each sequence runs
    block by block, the state and the conv history of one block starting the
    next.  Checkpoints are numbered sequence by sequence, in token order.

    Returns (o, finals, ckpts, where): o and finals as ``prefill``; ckpts
    (n, len(heads), d_v, d_k); where[i] = (s, p), checkpoint i taken after p
    tokens of sequence s.
    """
    if every <= 0:
        raise ValueError("every must be positive")
    N = x.shape[0]
    H = geom.n_v_heads
    heads = np.arange(H) if heads is None else np.asarray(heads)
    o = np.empty((N, len(heads), geom.d_v), F64)
    finals, ckpts, where = [], [], []
    for s in range(len(cu_seqlens) - 1):
        t0, t1 = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        if has_init[s]:
            S_full, hist = np.array(S0s[s], F64), np.asarray(hist0s[s], F64)
        else:
            S_full = np.zeros((H, geom.d_v, geom.d_k), F64)
            hist = np.zeros((max(geom.conv_width - 1, 0), geom.conv_channels), F64)
        S_heads = S_full[heads]
        for p0 in range(t0, t1, every):
            p1 = min(p0 + every, t1)
            o[p0:p1], S_heads, hist = layer_sequence(geom, x[p0:p1], a[p0:p1], b[p0:p1],
                                                     conv_w, S_full, hist, heads=heads)
            S_full = np.zeros((H, geom.d_v, geom.d_k), F64)
            S_full[heads] = S_heads
            if p1 - p0 == every:
                ckpts.append(np.array(S_heads))
                where.append((s, p1 - t0))
        finals.append((S_heads, hist))
    ck = (np.stack(ckpts) if ckpts
          else np.zeros((0, len(heads), geom.d_v, geom.d_k), F64))
    return o, finals, ck, where


# ----------------------------------------------------------------------------
# Chunked (WY / UT-transform) form -- used only to pin the sequential form.
# ----------------------------------------------------------------------------

def chunked_recurrence(q, k, v, g, beta, S0, chunk, q_scale=1.0):
    """The same recurrence computed chunk by chunk.

    Inside a chunk with cumulative log-gates G_r = sum_{j<=r} g_j:
      L_rj = beta_r e^{G_r - G_j} (k_r . k_j) for r > j (else 0),
      U = (I + L)^{-1} diag(beta) (V - diag(e^G) K S^T),
      O = q_scale (diag(e^G) Q S^T + P U),  P_rj = e^{G_r - G_j} (q_r . k_j), j <= r,
      S <- e^{G_last} S + (diag(e^{G_last - G}) U)^T K.
    q, k (T,H,d_k); v (T,H,d_v); g, beta (T,H); S0 (H,d_v,d_k).
    """
    T, H, dk = q.shape
    S = np.array(S0, F64)
    o = np.empty((T, H, v.shape[2]), F64)
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        n = c1 - c0
        for h in range(H):
            Q, K, V = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h]
            G = np.cumsum(np.asarray(g[c0:c1, h], F64))
            bt = np.asarray(beta[c0:c1, h], F64)
            D = G[:, None] - G[None, :]
            strict = np.tril(np.ones((n, n), bool), -1)
            causal = np.tril(np.ones((n, n), bool), 0)
            E = np.where(causal, np.exp(np.where(causal, D, 0.0)), 0.0)
            L = np.where(strict, bt[:, None] * E * (K @ K.T), 0.0)
            rhs = bt[:, None] * (V - np.exp(G)[:, None] * (K @ S[h].T))
            if _solve_tri is not None:
                U = _solve_tri(np.eye(n) + L, rhs, lower=True, unit_diagonal=True)
            else:
                U = np.linalg.solve(np.eye(n) + L, rhs)
            P = np.where(causal, E * (Q @ K.T), 0.0)
            o[c0:c1, h] = q_scale * (np.exp(G)[:, None] * (Q @ S[h].T) + P @ U)
            decay = np.exp(G[-1] - G)
            S[h] = np.exp(G[-1]) * S[h] + (decay[:, None] * U).T @ K
    return o, S


def frontend_sequence(geom, x, conv_w, hist0):
    """Front end of a whole sequence: per-token (q, k, v) expanded to v-heads.

    Returns q, k (T,H_v,d_k) and v (T,H_v,d_v).  A helper for the chunked
    self-check, built from ``frontend`` token by token.
    """
    x = np.asarray(x, F64)
    T = x.shape[0]
    W = geom.conv_width
    hist = np.asarray(hist0, F64).reshape(max(W - 1, 0), geom.conv_channels)
    qs = np.empty((T, geom.n_v_heads, geom.d_k))
    ks = np.empty((T, geom.n_v_heads, geom.d_k))
    vs = np.empty((T, geom.n_v_heads, geom.d_v))
    for t in range(T):
        window = np.concatenate([hist, x[t:t + 1]], axis=0)
        q, k, v = frontend(window, conv_w, geom)
        qs[t], ks[t], vs[t] = expand_heads(q, geom), expand_heads(k, geom), v
        if W > 1:
            hist = window[1:]
    return qs, ks, vs


def state_bytes(geom, n_slots=1):
    """Bytes of the fp32 recurrent state of ``n_slots`` slots (one layer)."""
    return 4 * n_slots * geom.n_v_heads * geom.d_v * geom.d_k


def conv_history_bytes(geom, elem_bytes):
    """Bytes of the W-1 rows of conv history that a causal width-W conv keeps."""
    return elem_bytes * max(geom.conv_width - 1, 0) * geom.conv_channels
