"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each one.  This is what makes the pins worth trusting:
a dropped term, a wrong sign or index, or a transposed operand must not pass."""
import os
import types

import pytest

import oracle_pins
from oracle import gdn_oracle

SRC = open(gdn_oracle.__file__).read()

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("no_decay", "Sa = alpha[:, None, None] * S", "Sa = S"),
    ("decay_after_read", "Sak = np.einsum(\"hij,hj->hi\", Sa, k)",
     "Sak = np.einsum(\"hij,hj->hi\", S, k)"),
    ("wrong_sign_write", "+ beta[:, None, None] * v[:, :, None] * k[:, None, :]",
     "- beta[:, None, None] * v[:, :, None] * k[:, None, :]"),
    ("no_erase", "S_new = Sa - beta[:, None, None] * Sak[:, :, None] * k[:, None, :]",
     "S_new = Sa + 0 * Sak[:, :, None] * k[:, None, :]"),
    ("output_transposed", "o = q_scale * np.einsum(\"hij,hj->hi\", S_new, q)",
     "o = q_scale * np.einsum(\"hji,hj->hi\", S_new, q)"),
    ("output_old_state", "o = q_scale * np.einsum(\"hij,hj->hi\", S_new, q)",
     "o = q_scale * np.einsum(\"hij,hj->hi\", S, q)"),
    ("softplus_sign", "return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))",
     "return np.maximum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))"),
    ("beta_not_sigmoid", "return g, np.exp(g), sigmoid(b)", "return g, np.exp(g), sigmoid(-b)"),
    ("gate_sign", "g = -softplus(a)\n    return g", "g = softplus(-a)\n    return g"),
    ("conv_taps_reversed", "y = np.einsum(\"cj,jc->c\", w, window)",
     "y = np.einsum(\"cj,jc->c\", w[:, ::-1], window)"),
    ("no_silu", "return silu(y)\n", "return y\n"),
    ("norm_no_sqrt", "return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)",
     "return x / ((x * x).sum(axis=-1, keepdims=True) + eps)"),
    ("interleaved_groups", "return np.repeat(qk, geom.group, axis=0)",
     "return np.tile(qk, (geom.group, 1))"),
    ("qk_swapped", "q = y[:nq].reshape(geom.n_k_heads, geom.d_k)\n    k = y[nq:2 * nq]",
     "k = y[:nq].reshape(geom.n_k_heads, geom.d_k)\n    q = y[nq:2 * nq]"),
    ("history_not_shifted", "        if W > 1:\n            hist = window[1:]\n    return o, S, hist",
     "        if W > 1:\n            hist = window[:-1]\n    return o, S, hist"),
    ("rollback_off_by_one", "return np.array(snaps[accepted - 1]), np.array(hists[accepted - 1])",
     "return np.array(snaps[accepted - 1 if accepted < len(snaps) else accepted - 2]), "
     "np.array(hists[accepted - 1])"),
    ("checkpoint_partial_block", "            if p1 - p0 == every:\n",
     "            if p1 - p0 >= 1:\n"),
    ("checkpoint_history_reset", "conv_w, S_full, hist, heads=heads)",
     "conv_w, S_full, 0 * hist, heads=heads)"),
    ("checkpoint_position_relative_to_batch", "where.append((s, p1 - t0))",
     "where.append((s, p1))"),
    ("norm_without_conv", "if geom.l2norm_qk and geom.conv_width > 0:", "if True:"),
    ("silu_without_conv", "y = np.asarray(window[-1], F64)", "y = silu(np.asarray(window[-1], F64))"),
    ("matrix_form_no_beta", "M = np.eye(dk) - beta[h] * np.outer(k[h], k[h])",
     "M = np.eye(dk) - np.outer(k[h], k[h])"),
    ("matrix_form_transposed", "out_S[h] = np.exp(g[h]) * (S[h] @ M)", "out_S[h] = np.exp(g[h]) * (M @ S[h])"),
    ("state_bytes_fp16", "return 4 * n_slots * geom.n_v_heads", "return 2 * n_slots * geom.n_v_heads"),
]


def _mutant(old, new):
    assert SRC.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = SRC.replace(old, new, 1)
    mod = types.ModuleType("gdn_oracle_mutant")
    mod.__file__ = os.path.join(os.path.dirname(gdn_oracle.__file__), "mutant.py")
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {name} passed every pin"
