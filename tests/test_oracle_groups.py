"""The per-k-head-group split of the oracle's prefill (used by the full-size
GPU parity tests) against the oracle run on the whole problem."""
import dataclasses

import numpy as np

import gdn_inputs as gi
from oracle import gdn_oracle as orc
from oracle import groups as OG


def _whole(g, inp, heads=None):
    S0 = np.stack([inp["state"][s] for s in inp["slots"]])
    h0 = np.stack([inp["hist"][s] for s in inp["slots"]])
    return orc.prefill(g, inp["x"], inp["a"], inp["b"], inp["conv_w"], inp["cu_seqlens"], S0, h0,
                       inp["has_init"], heads=heads)


def test_group_split_equals_whole_problem():
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, d_k=16, d_v=16, n_slots=4)
    inp = gi.prefill_inputs(seed=31, geom=g, lengths=[40, 0, 23], init_state=True, a_mean=-2.0)
    inp["has_init"] = np.array([1, 0, 1], np.int32)
    o_w, fin_w = _whole(g, inp)
    o_g, fin_g, heads = OG.prefill_by_groups(g, inp, workers=2)
    assert heads == list(range(6))
    assert np.allclose(o_g, o_w, rtol=0, atol=1e-12)
    for (S_g, h_g), (S_w, h_w) in zip(fin_g, fin_w):
        assert np.allclose(S_g, S_w, rtol=0, atol=1e-12)
        assert np.array_equal(h_g, h_w)


def test_group_split_head_subset():
    """One v-head per group: the heads come back in group order, and only the
    channels those heads read carry a history (the rest is NaN)."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, d_k=16, d_v=16, n_slots=3)
    inp = gi.prefill_inputs(seed=32, geom=g, lengths=[30, 17], init_state=True)
    o_g, fin_g, heads = OG.prefill_by_groups(g, inp, heads_of_group=lambda kh: [3 * kh + 2], workers=2)
    assert heads == [2, 5]
    o_w, fin_w = _whole(g, inp, heads=heads)
    assert np.allclose(o_g, o_w, rtol=0, atol=1e-12)
    for (S_g, h_g), (S_w, h_w) in zip(fin_g, fin_w):
        assert np.allclose(S_g, S_w, rtol=0, atol=1e-12)
        read = np.concatenate([OG.channels(g, 0, [2]), OG.channels(g, 1, [5])])
        assert np.array_equal(h_g[:, read], h_w[:, read])
        assert np.isnan(np.delete(h_g, read, axis=1)).all()
