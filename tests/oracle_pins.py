"""Pins of the fp64 oracle: facts fixed by the pages and by mathematics.

Every pin is a function ``pin_xxx(m)`` taking the oracle module, so the same
pins run against the real oracle (test_oracle_pins.py) and against copies of
it with a mistake planted (test_oracle_mutations.py), which must fail at
least one pin.  None of them re-types the oracle's formula: each compares it
with a closed form, a library routine, an independent derivation (the
chunked form), a printed number, or an invariant.
"""
from __future__ import annotations

import dataclasses
import json
import os

import numpy as np
import scipy.special

import gdn_inputs as gi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(rng, *shape):
    x = rng.normal(size=shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# scalar laws against library routines
# --------------------------------------------------------------------------

def pin_softplus_library(m):
    x = np.concatenate([np.linspace(-60, 60, 2001), [-700.0, 700.0, 0.0]])
    _close(m.softplus(x), np.logaddexp(0.0, x), 1e-15, "softplus vs logaddexp")


def pin_sigmoid_library(m):
    x = np.linspace(-80, 80, 3001)
    ref = scipy.special.expit(x)
    got = m.sigmoid(x)
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-300)) < 1e-13, "sigmoid vs expit"


def pin_gates_library(m):
    a = np.linspace(-20, 20, 401)
    b = np.linspace(-20, 20, 401)
    g, alpha, beta = m.gates(a, b)
    _close(alpha, scipy.special.expit(-a), 1e-14, "alpha = exp(-softplus(a)) = sigmoid(-a)")
    _close(g, np.log(scipy.special.expit(-a)), 1e-13, "g = log alpha")
    _close(beta, scipy.special.expit(b), 1e-15, "beta = sigmoid(b)")


def pin_silu_special(m):
    assert m.silu(0.0) == 0.0
    assert abs(m.silu(50.0) - 50.0) < 1e-12
    assert abs(m.silu(-50.0)) < 1e-18
    x = np.linspace(-10, 10, 201)
    _close(m.silu(x), x * scipy.special.expit(x), 1e-15, "silu vs x*expit(x)")


def pin_l2norm_library(m):
    rng = _rng(11)
    x = rng.normal(size=(5, 7, 128))
    _close(m.l2norm(x, 0.0), x / np.linalg.norm(x, axis=-1, keepdims=True), 1e-15,
           "l2norm vs numpy norm")
    # eps enters under the square root: zero vector stays zero, tiny vector is damped
    z = m.l2norm(np.zeros((1, 4)), 1e-6)
    assert np.all(z == 0.0)
    y = m.l2norm(np.full((1, 4), 1e-4), 1e-6)
    _close(y, np.full((1, 4), 1e-4 / np.sqrt(4e-8 + 1e-6)), 1e-14, "eps under sqrt")


# --------------------------------------------------------------------------
# conv front end
# --------------------------------------------------------------------------

def pin_conv_taps(m):
    rng = _rng(12)
    C, W = 6, 4
    window = rng.normal(size=(W, C))
    e_last = np.zeros((C, W))
    e_last[:, W - 1] = 1.0
    _close(m.conv_silu(window, e_last), window[-1] * scipy.special.expit(window[-1]), 1e-15,
           "w = e_{W-1} picks the current token")
    e_first = np.zeros((C, W))
    e_first[:, 0] = 1.0
    _close(m.conv_silu(window, e_first), window[0] * scipy.special.expit(window[0]), 1e-15,
           "w = e_0 picks the oldest token")


def pin_conv_library(m):
    """Causal depthwise conv over a sequence equals numpy's full convolution, cut."""
    rng = _rng(13)
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=1, d_k=2, d_v=2,
                               l2norm_qk=False)
    C, W, T = geom.conv_channels, geom.conv_width, 9
    x = rng.normal(size=(T, C))
    w = rng.normal(size=(C, W))
    hist = np.zeros((W - 1, C))
    for t in range(T):
        window = np.concatenate([hist, x[t:t + 1]])
        y = m.conv_silu(window, w)
        for c in range(C):
            full = np.convolve(x[:, c], w[c, ::-1])  # causal cross-correlation
            ref = full[t]
            _close(y[c], ref * scipy.special.expit(ref), 1e-14, "conv vs np.convolve")
        hist = window[1:]


def pin_frontend_split_and_norm(m):
    """Channel order q | k | v (head-major) and unit-length q, k after the norm."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=4, d_k=4, d_v=3)
    C, W = geom.conv_channels, geom.conv_width
    assert C == 2 * 2 * 4 + 4 * 3
    window = np.zeros((W, C))
    window[-1] = np.arange(1, C + 1, dtype=np.float64)
    w = np.zeros((C, W))
    w[:, -1] = 1.0
    q, k, v = m.frontend(window, w, geom)
    silu = lambda z: z * scipy.special.expit(z)  # noqa: E731
    ch = np.arange(1, C + 1, dtype=np.float64)
    yq = silu(ch[:8]).reshape(2, 4)
    yk = silu(ch[8:16]).reshape(2, 4)
    _close(q, yq / np.linalg.norm(yq, axis=1, keepdims=True), 1e-7, "q channels and norm")
    _close(k, yk / np.linalg.norm(yk, axis=1, keepdims=True), 1e-7, "k channels and norm")
    _close(v, silu(ch[16:]).reshape(4, 3), 1e-15, "v channels, no norm")


def pin_head_grouping(m):
    """v-head h reads k-head floor(h / (H_v/H_k)) (contiguous groups)."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6)
    qk = np.array([[1.0, 0.0], [0.0, 1.0]])
    ex = m.expand_heads(qk, geom)
    assert ex.shape == (6, 2)
    assert np.array_equal(ex[:, 1], [0, 0, 0, 1, 1, 1])


def pin_conv_history(m):
    """After L tokens the history holds the last W-1 inputs, oldest first,
    mixing the initial history when L < W-1."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=1, d_k=2, d_v=2)
    C, W = geom.conv_channels, geom.conv_width
    rng = _rng(14)
    h0 = rng.normal(size=(W - 1, C))
    w = rng.normal(size=(C, W))
    for L in (1, 2, 3, 4, 9):
        x = rng.normal(size=(L, C))
        a = rng.normal(size=(L, 1))
        b = rng.normal(size=(L, 1))
        _, _, hist = m.layer_sequence(geom, x, a, b, w, np.zeros((1, 2, 2)), h0)
        ref = np.concatenate([h0, x])[-(W - 1):]
        assert np.array_equal(hist, ref), f"history after {L} tokens"


# --------------------------------------------------------------------------
# the delta rule: closed forms, invariants, independent forms
# --------------------------------------------------------------------------

def pin_expanded_equals_matrix_form(m):
    """The expanded step (no d_k x d_k matrix) equals the step with the
    transition matrix (I - beta k k^T) formed explicitly, the rule as written;
    the transition's own action is pinned by pin_transition_action."""
    rng = _rng(21)
    H, d = 3, 5
    S = rng.normal(size=(H, d, d))
    q, k = rng.normal(size=(H, d)), 1.7 * _unit(rng, H, d)
    v = rng.normal(size=(H, d))
    g = -rng.uniform(0, 2, size=H)
    beta = rng.uniform(0, 1, size=H)
    S1, o1 = m.delta_rule_step(S, q, k, v, g, beta, 0.7)
    S2, o2 = m.delta_rule_step_matrix(S, q, k, v, g, beta, 0.7)
    _close(S1, S2, 1e-14, "expanded vs matrix form: S_t")
    _close(o1, o2, 1e-14, "expanded vs matrix form: o_t")


def pin_transition_action(m):
    """For a unit key the transition I - beta k k^T scales k by (1 - beta) and
    leaves every direction orthogonal to k alone, so
        S_t k = alpha (1 - beta) S_{t-1} k + beta v,   S_t u = alpha S_{t-1} u  (u . k = 0),
        o_t = q_scale S_t q  (linear in q).
    Checked on both the expanded and the matrix form of the step."""
    rng = _rng(35)
    H, d = 3, 6
    for step in (m.delta_rule_step, m.delta_rule_step_matrix):
        S = rng.normal(size=(H, d, d))
        k = _unit(rng, H, d)
        q = rng.normal(size=(H, d))
        v = rng.normal(size=(H, d))
        g = -rng.uniform(0, 2, size=H)
        beta = rng.uniform(0, 1, size=H)
        S1, o1 = step(S, q, k, v, g, beta, 0.3)
        alpha = np.exp(g)
        Sk = np.einsum("hij,hj->hi", S, k)
        _close(np.einsum("hij,hj->hi", S1, k),
               (alpha * (1 - beta))[:, None] * Sk + beta[:, None] * v, 1e-13,
               f"{step.__name__}: action on k")
        u = rng.normal(size=(H, d))
        u -= (u * k).sum(1, keepdims=True) * k  # orthogonal to k
        _close(np.einsum("hij,hj->hi", S1, u), alpha[:, None] * np.einsum("hij,hj->hi", S, u), 1e-13,
               f"{step.__name__}: action orthogonal to k")
        _, o2 = step(S, 2.0 * q, k, v, g, beta, 0.3)
        _close(o2, 2.0 * o1, 1e-14, f"{step.__name__}: o linear in q")
        _close(o1, 0.3 * np.einsum("hij,hj->hi", S1, q), 1e-14, f"{step.__name__}: o from the new state")


def pin_no_conv_front_end(m):
    """Without the conv front end (conv_width = 0, the tiny workload's layout)
    x holds q | k | v and the layer applies nothing to them: no conv, no SiLU,
    no norm.  Keys and queries of arbitrary length show any of those:
      - first token from a zero state: S_1 = beta v k^T, o_1 = beta (k . q) v;
      - beta = 0: o_t = e^{sum_{s<=t} g_s} S_0 q_t (linear in the raw q);
      - a whole sequence equals the plain recurrence on the split x."""
    geom = dataclasses.replace(gi.GEOM_TINY, n_k_heads=2, n_v_heads=4, d_k=5, d_v=3)
    rng = _rng(36)
    Hk, Hv, dk, dv = 2, 4, 5, 3
    T = 7
    q = 2.5 * rng.normal(size=(T, Hk, dk))
    k = 0.6 * rng.normal(size=(T, Hk, dk))
    v = rng.normal(size=(T, Hv, dv))
    x = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    a = rng.normal(size=(T, Hv))
    b = rng.normal(size=(T, Hv))
    w = np.zeros((geom.conv_channels, 0))
    hist = np.zeros((0, geom.conv_channels))
    grp = Hv // Hk
    qh, kh = np.repeat(q, grp, axis=1), np.repeat(k, grp, axis=1)
    beta = scipy.special.expit(b)
    g = -np.logaddexp(0.0, a)
    # first token from zero
    o, S, _ = m.layer_sequence(geom, x[:1], a[:1], b[:1], w, np.zeros((Hv, dv, dk)), hist)
    _close(S, beta[0][:, None, None] * v[0][:, :, None] * kh[0][:, None, :], 1e-15, "W=0 first-token state")
    _close(o[0], (beta[0] * (kh[0] * qh[0]).sum(1))[:, None] * v[0], 1e-14, "W=0 first-token output")
    # beta = 0 over the sequence
    S0 = rng.normal(size=(Hv, dv, dk))
    b0 = np.full_like(b, -1000.0)
    o, S, _ = m.layer_sequence(geom, x, a, b0, w, S0, hist)
    G = np.cumsum(g, axis=0)
    for t in range(T):
        _close(o[t], np.exp(G[t])[:, None] * np.einsum("hij,hj->hi", S0, qh[t]), 1e-13, f"W=0 beta=0 t={t}")
    # the whole layer equals the recurrence on the split input
    o, S, _ = m.layer_sequence(geom, x, a, b, w, S0, hist)
    o2, S2 = m.recurrence(qh, kh, v, g, beta, S0)
    _close(o, o2, 1e-14, "W=0 layer vs recurrence: o")
    _close(S, S2, 1e-14, "W=0 layer vs recurrence: S")


def pin_beta_zero(m):
    """beta = 0: S_t = alpha_t S_{t-1}, o_t = e^{sum_{s<=t} g_s} S_0 q_t."""
    rng = _rng(22)
    T, H, d = 17, 2, 6
    S0 = rng.normal(size=(H, d, d))
    q, k = _unit(rng, T, H, d), _unit(rng, T, H, d)
    v = rng.normal(size=(T, H, d))
    g = -rng.uniform(0, 0.5, size=(T, H))
    o, S = m.recurrence(q, k, v, g, np.zeros((T, H)), S0)
    G = np.cumsum(g, axis=0)
    for t in range(T):
        ref = np.exp(G[t])[:, None] * np.einsum("hij,hj->hi", S0, q[t])
        _close(o[t], ref, 1e-13, f"beta=0 output t={t}")
    _close(S, np.exp(G[-1])[:, None, None] * S0, 1e-13, "beta=0 final state")


def pin_unit_key_write(m):
    """alpha = beta = 1 and unit k: the write is exact, S_t k_t = v_t."""
    rng = _rng(23)
    T, H, d = 12, 2, 8
    S = rng.normal(size=(H, d, d))
    for t in range(T):
        k = _unit(rng, H, d)
        v = rng.normal(size=(H, d))
        q = _unit(rng, H, d)
        S, _ = m.delta_rule_step(S, q, k, v, np.zeros(H), np.ones(H))
        _close(np.einsum("hij,hj->hi", S, k), v, 1e-12, "S_t k_t = v_t")


def pin_orthonormal_keys(m):
    """alpha = beta = 1, orthonormal k_1..k_n:
    S_n = S_0 (I - sum k k^T) + sum v k^T, whatever the order."""
    rng = _rng(24)
    d, n = 8, 5
    Qm, _ = np.linalg.qr(rng.normal(size=(d, d)))
    keys = Qm[:, :n].T
    vals = rng.normal(size=(n, d))
    S0 = rng.normal(size=(1, d, d))
    ref = S0[0] @ (np.eye(d) - keys.T @ keys) + vals.T @ keys
    for order in (range(n), reversed(range(n)), [2, 0, 4, 1, 3]):
        order = list(order)
        q = _unit(rng, n, 1, d)
        _, S = m.recurrence(q, keys[order][:, None, :], vals[order][:, None, :],
                            np.zeros((n, 1)), np.ones((n, 1)), S0)
        _close(S[0], ref, 1e-13, f"orthonormal keys order {order}")


def pin_first_token(m):
    """From a zero state: S_1 = beta v k^T and o_1 = beta (k . q) v."""
    rng = _rng(25)
    H, d = 4, 7
    q, k = _unit(rng, H, d), _unit(rng, H, d)
    v = rng.normal(size=(H, d))
    g = -rng.uniform(0, 3, size=H)
    beta = rng.uniform(0, 1, size=H)
    S, o = m.delta_rule_step(np.zeros((H, d, d)), q, k, v, g, beta)
    _close(S, beta[:, None, None] * v[:, :, None] * k[:, None, :], 1e-15, "S_1")
    _close(o, (beta * (k * q).sum(1))[:, None] * v, 1e-14, "o_1")


def pin_homogeneity(m):
    """(S_0, v) -> c (S_0, v) scales (S_t, o_t) by c."""
    rng = _rng(26)
    T, H, d = 9, 2, 6
    S0 = rng.normal(size=(H, d, d))
    q, k = _unit(rng, T, H, d), _unit(rng, T, H, d)
    v = rng.normal(size=(T, H, d))
    g = -rng.uniform(0, 1, size=(T, H))
    beta = rng.uniform(0, 1, size=(T, H))
    o1, S1 = m.recurrence(q, k, v, g, beta, S0)
    o2, S2 = m.recurrence(q, k, 3.0 * v, g, beta, 3.0 * S0)
    _close(o2, 3.0 * o1, 1e-14, "homogeneous o")
    _close(S2, 3.0 * S1, 1e-14, "homogeneous S")


def pin_norm_bound(m):
    """Unit k, beta in [0,1]: ||S_t||_2 <= alpha_t ||S_{t-1}||_2 + beta_t ||v_t||."""
    rng = _rng(27)
    H, d = 3, 6
    S = rng.normal(size=(H, d, d))
    for _ in range(30):
        q, k = _unit(rng, H, d), _unit(rng, H, d)
        v = rng.normal(size=(H, d))
        g = -rng.uniform(0, 1, size=H)
        beta = rng.uniform(0, 1, size=H)
        S1, _ = m.delta_rule_step(S, q, k, v, g, beta)
        for h in range(H):
            lhs = np.linalg.norm(S1[h], 2)
            rhs = np.exp(g[h]) * np.linalg.norm(S[h], 2) + beta[h] * np.linalg.norm(v[h])
            assert lhs <= rhs * (1 + 1e-12), "spectral-norm bound"
        S = S1


def pin_chunked_equals_sequential(m):
    """An independent derivation (WY/UT chunked form) agrees with the sequential rule."""
    rng = _rng(28)
    cases = 0
    for d in (2, 4, 16):
        for G in (1, 3):
            for T in (1, 2, 3, 5, 63, 64, 65, 130):
                for chunk in (1, 2, 4, 16, 64, 1000):
                    if (d == 16 and T > 65 and chunk < 16) or (T > 64 and chunk == 1 and d > 2):
                        continue
                    Hk = 2
                    H = Hk * G
                    qk = _unit(rng, T, Hk, d)
                    kk = _unit(rng, T, Hk, d)
                    q = np.repeat(qk, G, axis=1)
                    k = np.repeat(kk, G, axis=1)
                    v = rng.normal(size=(T, H, d + 1))
                    long_memory = (cases % 2 == 1)
                    a = rng.normal(-6.0 if long_memory else 0.0, 1.0, size=(T, H))
                    g = -np.logaddexp(0.0, a)
                    beta = scipy.special.expit(rng.normal(size=(T, H)))
                    S0 = 0.1 * rng.normal(size=(H, d + 1, d))
                    o1, S1 = m.recurrence(q, k, v, g, beta, S0, 0.5)
                    o2, S2 = m.chunked_recurrence(q, k, v, g, beta, S0, chunk, 0.5)
                    _close(o1, o2, 1e-11, f"o d={d} G={G} T={T} chunk={chunk}")
                    _close(S1, S2, 1e-11, f"S d={d} G={G} T={T} chunk={chunk}")
                    cases += 1
    assert cases > 200


def pin_state_size_independent_of_T(m):
    """[Hybrid] section 3: the state has the same size at any context length."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=2, d_k=4, d_v=4)
    rng = _rng(29)
    shapes = set()
    for T in (1, 7, 300):
        x = rng.normal(size=(T, geom.conv_channels))
        a = rng.normal(size=(T, 2))
        b = rng.normal(size=(T, 2))
        w = rng.normal(size=(geom.conv_channels, 4))
        _, S, hist = m.layer_sequence(geom, x, a, b, w, np.zeros((2, 4, 4)),
                                      np.zeros((3, geom.conv_channels)))
        shapes.add((S.shape, hist.shape))
    assert len(shapes) == 1


def pin_page_byte_counts(m):
    """Printed byte counts of the pages reproduced from the geometry."""
    with open(os.path.join(GOLDEN, "page_sizes.json")) as f:
        pg = json.load(f)
    g4b = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=16, n_v_heads=32, d_k=128, d_v=128)
    ssm = m.state_bytes(g4b)
    assert ssm == pg["hybrid_4b_ssm_state_bytes"]["value"]
    # conv part: W-1 = 3 rows of history; 49152 B = 3 rows x 8192 channels x 2 B
    g4b_conv = dataclasses.replace(g4b, n_k_heads=16, n_v_heads=32, d_k=128, d_v=128)
    ch = g4b_conv.conv_channels
    assert ch == 2 * 16 * 128 + 32 * 128 == 8192
    conv = m.conv_history_bytes(g4b_conv, 2)
    assert conv == pg["hybrid_4b_conv_bytes"]["value"]
    total = ssm + conv
    assert total == pg["hybrid_4b_layer_state_bytes"]["value"]
    assert total % pg["hybrid_4b_layer_state_bytes"]["attention_page_bytes_per_token"] == 0
    assert total // 4096 == pg["hybrid_4b_layer_state_bytes"]["tokens_for_equal_page"]
    snap = pg["hybrid_4b_gdn_layers"]["value"] * total / 2**20
    assert abs(snap - pg["hybrid_4b_gdn_layers"]["snapshot_mb"]) < 0.05
    assert abs(total / 2**20 - pg["hybrid_4b_state_mb"]["value"]) < 0.005
    sg = pg["strata_geometry"]
    geo = gi.GEOM_QWEN
    assert geo.conv_channels == sg["ssm_conv_channels"]
    assert geo.n_v_heads * geo.d_v == sg["ssm_value_dim"]
    assert (geo.n_k_heads, geo.n_v_heads, geo.d_k, geo.conv_width) == (
        sg["ssm_k_heads"], sg["ssm_v_heads"], sg["ssm_state_size"], sg["ssm_d_conv"])
    # the layer of this geometry keeps 48 x 128 x 128 fp32 per slot
    assert m.state_bytes(geo) == 3145728


def pin_verify_rollback_replay(m):
    """rollback(a) equals running the layer over the first a drafts."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, d_k=8, d_v=8)
    rng = _rng(30)
    C = geom.conv_channels
    kd = 4
    S0 = rng.normal(size=(6, 8, 8)) * 0.1
    h0 = rng.normal(size=(3, C)) * 0.1
    x = rng.normal(size=(kd, C))
    a = rng.normal(size=(kd, 6))
    b = rng.normal(size=(kd, 6))
    w = rng.normal(size=(C, 4)) * 0.5
    o, snaps, hists = m.verify(geom, S0, h0, x, a, b, w)
    for acc in range(kd + 1):
        S_r, h_r = m.rollback(S0, h0, snaps, hists, acc)
        o_ref, S_ref, h_ref = m.layer_sequence(geom, x[:acc], a[:acc], b[:acc], w, S0, h0)
        _close(S_r, S_ref, 1e-14, f"rollback state a={acc}")
        assert np.array_equal(h_r, h_ref)
        if acc:
            _close(o[:acc], o_ref, 1e-14, "verify outputs")


def pin_decode_touches_only_its_slots(m):
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=2, d_k=4, d_v=4,
                               n_slots=5)
    rng = _rng(31)
    C = geom.conv_channels
    st = rng.normal(size=(5, 2, 4, 4))
    hi = rng.normal(size=(5, 3, C))
    x = rng.normal(size=(2, C))
    a = rng.normal(size=(2, 2))
    b = rng.normal(size=(2, 2))
    w = rng.normal(size=(C, 4))
    _, st2, hi2 = m.decode_step(geom, st, hi, x, a, b, w, [3, 1])
    for s in (0, 2, 4):
        assert np.array_equal(st2[s], st[s]) and np.array_equal(hi2[s], hi[s])
    assert not np.array_equal(st2[3], st[3])


def pin_prefill_is_per_sequence(m):
    """Varlen prefill of two sequences equals each sequence run alone, and a
    sequence split in two (second part starting from the first's final state
    and history) equals the whole sequence."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=3, d_k=4, d_v=4)
    rng = _rng(32)
    C = geom.conv_channels
    N = 23
    x = rng.normal(size=(N, C))
    a = rng.normal(size=(N, 3))
    b = rng.normal(size=(N, 3))
    w = rng.normal(size=(C, 4))
    S0 = rng.normal(size=(2, 3, 4, 4))
    h0 = rng.normal(size=(2, 3, C))
    cu = [0, 9, 23]
    o, fin = m.prefill(geom, x, a, b, w, cu, S0, h0, [1, 0])
    o1, S1, hh1 = m.layer_sequence(geom, x[:9], a[:9], b[:9], w, S0[0], h0[0])
    _close(o[:9], o1, 1e-15, "seq 0 alone")
    z = np.zeros_like(S0[0])
    o2a, S2a, h2a = m.layer_sequence(geom, x[9:15], a[9:15], b[9:15], w, z, np.zeros((3, C)))
    o2b, S2b, h2b = m.layer_sequence(geom, x[15:], a[15:], b[15:], w, S2a, h2a)
    _close(o[9:15], o2a, 1e-14, "seq 1 first part")
    _close(o[15:], o2b, 1e-13, "seq 1 continued from its state")
    _close(fin[1][0], S2b, 1e-13, "seq 1 final state")



def _ckpt_case(rng, geom, lens, has_init):
    C, H = geom.conv_channels, geom.n_v_heads
    N = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    x = rng.normal(size=(N, C))
    a = rng.normal(-1.0, 1.0, size=(N, H))
    b = rng.normal(size=(N, H))
    w = rng.normal(size=(C, geom.conv_width))
    S0 = 0.5 * rng.normal(size=(len(lens), H, geom.d_v, geom.d_k))
    h0 = rng.normal(size=(len(lens), geom.conv_width - 1, C))
    return cu, x, a, b, w, S0, h0


def pin_checkpoints_beta_zero(m):
    """beta = 0 (b far below zero): checkpoint after p tokens = e^{sum_{t<p} g_t} S_0,
    which fixes both the positions and the count of the checkpoints."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=2, d_k=4, d_v=4)
    rng = _rng(33)
    lens, every = [13, 0, 8, 4], 4
    cu, x, a, b, w, S0, h0 = _ckpt_case(rng, geom, lens, [1, 0, 1, 0])
    b[:] = -1000.0
    o, fin, ck, where = m.prefill_checkpoints(geom, x, a, b, w, cu, S0, h0, [1, 0, 1, 0], every)
    want = [(s, p) for s, n in enumerate(lens) for p in range(every, n + 1, every)]
    assert where == want, (where, want)
    assert ck.shape == (len(want), 2, 4, 4)
    g = -np.logaddexp(0.0, a)
    for i, (s, p) in enumerate(want):
        start = S0[s] if s in (0, 2) else np.zeros_like(S0[s])
        ref = np.exp(g[cu[s]:cu[s] + p].sum(axis=0))[:, None, None] * start
        _close(ck[i], ref, 1e-13, f"beta=0 checkpoint {i} (seq {s}, p {p})")


def pin_checkpoints_chunked_prefix(m):
    """Checkpoint after p tokens equals the chunked form (an independent
    derivation) run over the first p tokens with the front end applied; a
    sequence whose length is a multiple of the block ends on a checkpoint equal
    to its final state; outputs equal the plain prefill's."""
    geom = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=3, d_k=4, d_v=4)
    rng = _rng(34)
    lens, every, init = [14, 10, 5], 5, [1, 0, 1]
    cu, x, a, b, w, S0, h0 = _ckpt_case(rng, geom, lens, init)
    heads = [2, 0]
    o, fin, ck, where = m.prefill_checkpoints(geom, x, a, b, w, cu, S0, h0, init, every,
                                              heads=heads)
    assert [p for _, p in where] == [5, 10, 5, 10, 5]
    oref, finref = m.prefill(geom, x, a, b, w, cu, S0, h0, init, heads=heads)
    _close(o, oref, 1e-13, "outputs vs plain prefill")
    g, _, beta = m.gates(a, b)
    for i, (s, p) in enumerate(where):
        t0 = cu[s]
        start = S0[s] if init[s] else np.zeros_like(S0[s])
        hist = h0[s] if init[s] else np.zeros_like(h0[s])
        q, k, v = m.frontend_sequence(geom, x[t0:t0 + p], w, hist)
        _, Sc = m.chunked_recurrence(q[:, heads], k[:, heads], v[:, heads], g[t0:t0 + p][:, heads],
                                     beta[t0:t0 + p][:, heads], start[heads], 3, geom.q_scale)
        _close(ck[i], Sc, 1e-11, f"checkpoint {i} (seq {s}, p {p}) vs chunked prefix")
        if p == lens[s]:
            _close(ck[i], fin[s][0], 1e-15, f"seq {s} ends on its last checkpoint")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
