"""Chunked varlen prefill on the GPU against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import harness as H
from oracle import gdn_oracle as orc
from oracle import groups as OG

pytestmark = pytest.mark.gpu


def _gdn():
    import gated_deltanet_delta_amd as gdn
    gdn.lib()
    return gdn


def _prefill(g, inp, pool=None, ws=None):
    gdn = _gdn()
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    if pool is None:
        pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    N = inp["x"].shape[0]
    S = len(inp["cu_seqlens"]) - 1
    o = torch.zeros(N, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    if ws is None:
        ws = gdn.alloc_prefill_workspace(geom, N, S)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.prefill_chunked(geom, pool, H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt),
                        H.dev(inp["conv_w"]) if g.conv_width else None, H.dev(inp["cu_seqlens"]),
                        H.dev(inp["slots"]), H.dev(inp["has_init"]), o, ws, dev_err=err)
    torch.cuda.synchronize()
    return pool, o, int(err.item())


def _oracle(g, inp, heads=None):
    S = len(inp["cu_seqlens"]) - 1
    S0 = np.stack([inp["state"][s] for s in inp["slots"]])
    h0 = np.stack([inp["hist"][s] for s in inp["slots"]]) if g.conv_width else np.zeros((S, 0, g.conv_channels))
    return orc.prefill(g, inp["x"], inp["a"], inp["b"], inp["conv_w"], inp["cu_seqlens"], S0, h0,
                       inp["has_init"], heads=heads)


def _check(g, inp, pool, o, heads=None, tol=None, ref=None):
    """GPU results against the oracle (``ref`` = its (o, finals) for ``heads``
    when already computed, e.g. per k-head group in worker processes)."""
    tol = H.tol_for(g) if tol is None else tol
    heads_l = list(range(g.n_v_heads)) if heads is None else list(heads)
    o_ref, finals = _oracle(g, inp, heads=heads) if ref is None else ref
    cu = inp["cu_seqlens"]
    o_gpu = H.f64(o)[:, heads_l]
    state = pool.state.cpu().numpy()
    hist = H.read_hist(g, pool) if g.conv_width else None
    pos = H.positions(pool) if g.conv_width else None
    for s in range(len(cu) - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        if t1 > t0:
            e = H.relerr(o_gpu[t0:t1], o_ref[t0:t1])
            assert e <= tol, f"seq {s} output rel err {e:.3e}"
        slot = int(inp["slots"][s])
        e = H.relerr(state[slot][heads_l], finals[s][0])
        assert e <= tol, f"seq {s} final state rel err {e:.3e}"
        if g.conv_width:
            h_ref = finals[s][1]
            known = ~np.isnan(h_ref)  # channels the oracle was run on
            assert np.array_equal(hist[slot][known], h_ref[known].astype(np.float32)), f"seq {s} conv history"
            start = int(inp["pos"][slot]) if inp["has_init"][s] else 0
            assert pos[slot] == start + (t1 - t0)


def test_workload1_through_prefill_fp32():
    """Tiny fp32 recurrence via the chunked path (fp32 MFMA): 1e-4."""
    inp = gi.workload(1)
    g = inp["geom"]
    inp = dict(inp, state=np.zeros((1, 1, 16, 16), np.float32), hist=np.zeros((1, 0, g.conv_channels)),
               pos=np.zeros(1, np.int64))
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


@pytest.mark.parametrize("T", [1, 3, 63, 64, 65, 130, 200])
def test_prefill_small_lengths_bf16(T):
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=3)
    inp = gi.prefill_inputs(seed=200 + T, geom=g, lengths=[T])
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


@pytest.mark.parametrize("d", [16, 32, 64])
def test_prefill_other_head_sizes(d):
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=4, d_k=d, d_v=d, n_slots=4)
    inp = gi.prefill_inputs(seed=300 + d, geom=g, lengths=[150, 64, 1], init_state=True, a_mean=-2.0)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


def test_prefill_fp32_varlen_with_init():
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=3, d_k=32, d_v=32, n_slots=4,
                            dtype_in=gi.F32, dtype_out=gi.F32)
    inp = gi.prefill_inputs(seed=77, geom=g, lengths=[70, 129, 2], init_state=True)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


def test_prefill_varlen_ragged_with_empty_and_init():
    """Sequences of lengths 0, 1, 2, 64, 200 with and without initial state."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=6)
    inp = gi.prefill_inputs(seed=55, geom=g, lengths=[0, 1, 2, 64, 200], a_mean=-2.0)
    inp["has_init"] = np.array([1, 1, 0, 1, 0], np.int32)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


@pytest.mark.parametrize("lengths", [[65] * 9, [1] * 20, [1, 65, 129, 193, 1, 65, 129, 257]])
def test_prefill_chunk_count_at_its_bound(lengths):
    """Partitions whose chunk count equals the bound
    floor((n_tokens + 63 n_seqs) / 64) that sizes the plan."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=2, n_slots=len(lengths))
    inp = gi.prefill_inputs(seed=400 + len(lengths), geom=g, lengths=lengths, init_state=True, a_mean=-2.0)
    n = sum(lengths)
    assert sum((t + 63) // 64 for t in lengths) == (n + 63 * len(lengths)) // 64
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


@pytest.mark.parametrize("lengths", [[65, 0], [0, 1, 0], [64, 64, 0, 0]])
def test_prefill_trailing_empty_sequences(lengths):
    """Empty sequences after the last chunk: their chunk index equals the
    chunk-count bound, so nothing may be staged for them."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=2, n_slots=len(lengths))
    inp = gi.prefill_inputs(seed=410 + len(lengths), geom=g, lengths=lengths, init_state=True, a_mean=-2.0)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


def test_prefill_reused_workspace_sees_new_inputs():
    """Two different prefills back to back on one workspace: the second reads
    only what its own chunk kernel published."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=2)
    inp1 = gi.prefill_inputs(seed=501, geom=g, lengths=[300])
    inp2 = gi.prefill_inputs(seed=502, geom=g, lengths=[300])
    ws = gdn.alloc_prefill_workspace(H.to_geom(g), 300, 1)
    _prefill(g, inp1, ws=ws)
    pool, o, err = _prefill(g, inp2, ws=ws)
    assert err == 0
    _check(g, inp2, pool, o)


def test_prefill_segmented_launches():
    """32 k-heads with 8 v-heads each: more chain workgroups than one launch
    holds beside its producers (at most 24 per XCD, so 24 k-heads per
    launch), so the prefill runs as two launches over k-head ranges, the last
    one also writing the conv positions; heads on both sides of the split."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=32, n_v_heads=256, n_slots=2)
    inp = gi.prefill_inputs(seed=503, geom=g, lengths=[300, 70], init_state=True, a_mean=-2.0)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o, heads=[0, 100, 191, 192, 255])


@pytest.mark.parametrize("lengths", [[300, 0, 130, 64], [64, 1, 129]])
def test_prefill_one_launch_walks_the_sequences(lengths):
    """Several sequences in one chain launch: every chain workgroup takes the
    sequences in turn (an empty one in between, a one-token one), each from
    its own slot's initial state."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=len(lengths) + 1)
    inp = gi.prefill_inputs(seed=540 + len(lengths), geom=g, lengths=lengths, init_state=True, a_mean=-2.0)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o, heads=[0, 13, 47])


@pytest.mark.parametrize("G", [4, 8])
def test_prefill_bf16_more_v_heads_per_k_head(G):
    """More than three v-heads per k-head: a producer forms the inverses and
    T diag(beta) of its k-head's v-heads in groups, from K K^T kept in LDS,
    and G chains read one item."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=G, n_slots=2)
    inp = gi.prefill_inputs(seed=520 + G, geom=g, lengths=[150, 77], init_state=True, a_mean=-2.0)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o)


@pytest.mark.parametrize("n_v_heads,lengths", [(64, [70]), (64, [70, 20]), (32, [70, 20]), (80, [70, 20])])
def test_prefill_v_heads_per_k_head(n_v_heads, lengths):
    """16 k-heads with 4, 2 and 5 v-heads each: 8, 4 and 10 chain workgroups
    per XCD, the rest of the launch producing; one and two sequences."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=16, n_v_heads=n_v_heads, n_slots=len(lengths))
    inp = gi.prefill_inputs(seed=530 + n_v_heads + len(lengths), geom=g, lengths=lengths, init_state=True,
                            a_mean=-2.0)
    pool, o, err = _prefill(g, inp)
    assert err == 0
    _check(g, inp, pool, o, heads=[0, 5, n_v_heads - 1])


def test_prefill_then_decode_continues_the_sequence():
    """Prefill the first part of a sequence, decode the rest token by token:
    matches the oracle over the whole sequence."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=2)
    inp = gi.prefill_inputs(seed=66, geom=g, lengths=[100])
    pre = dict(inp, x=inp["x"][:90], a=inp["a"][:90], b=inp["b"][:90], cu_seqlens=np.array([0, 90], np.int32))
    pool, o, err = _prefill(g, pre)
    assert err == 0
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    slot = H.dev(inp["slots"])
    outs = [H.f64(o)]
    for t in range(90, 100):
        ot = torch.empty(1, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
        gdn.decode_step(geom, pool, H.dev(inp["x"][t:t + 1], dt), H.dev(inp["a"][t:t + 1], dt),
                        H.dev(inp["b"][t:t + 1], dt), H.dev(inp["conv_w"]), slot, ot)
        outs.append(H.f64(ot))
    o_all = np.concatenate(outs)
    o_ref, S_ref, h_ref = orc.layer_sequence(g, inp["x"], inp["a"], inp["b"], inp["conv_w"],
                                             np.zeros((g.n_v_heads, 128, 128)), np.zeros((3, g.conv_channels)))
    assert H.relerr(o_all, o_ref) <= H.TOL_BF16
    s = int(inp["slots"][0])
    assert H.relerr(pool.state.cpu().numpy()[s], S_ref) <= H.TOL_BF16
    assert np.array_equal(H.read_hist(g, pool)[s], h_ref.astype(np.float32))


def test_prefill_deterministic():
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=4, n_v_heads=12, n_slots=2)
    inp = gi.prefill_inputs(seed=88, geom=g, lengths=[300])
    p1, o1, _ = _prefill(g, inp)
    p2, o2, _ = _prefill(g, inp)
    assert torch.equal(o1, o2) and torch.equal(p1.state, p2.state)


def test_prefill_sequence_alone_equals_batched():
    """A sequence's outputs and final state do not depend on the other sequences of the batch."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=4)
    inp = gi.prefill_inputs(seed=99, geom=g, lengths=[77, 140, 33], init_state=True)
    pool, o, _ = _prefill(g, inp)
    cu = inp["cu_seqlens"]
    alone = dict(inp, x=inp["x"][cu[1]:cu[2]], a=inp["a"][cu[1]:cu[2]], b=inp["b"][cu[1]:cu[2]],
                 cu_seqlens=np.array([0, cu[2] - cu[1]], np.int32), slots=inp["slots"][1:2],
                 has_init=inp["has_init"][1:2])
    pool1, o1, _ = _prefill(g, alone)
    assert torch.equal(o[cu[1]:cu[2]], o1)
    s = int(inp["slots"][1])
    assert torch.equal(pool.state[s], pool1.state[s])


def test_prefill_bad_seqlens_reported():
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=3)
    inp = gi.prefill_inputs(seed=5, geom=g, lengths=[40, 30])
    inp["cu_seqlens"] = np.array([0, 50, 70], np.int32)  # last != N = 70? (valid) -> make it decreasing
    inp["cu_seqlens"] = np.array([0, 50, 45], np.int32)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    before = pool.state.clone()
    _, o, err = _prefill(g, inp, pool)
    assert err == gdn.DEV_BAD_SEQLENS
    assert torch.equal(pool.state, before)


def test_workload3_full_length_all_heads():
    """T = 8192, full geometry, every one of the 48 v-heads against the oracle
    (run per k-head group in worker processes); every conv channel's history."""
    inp = gi.workload(3)
    g = inp["geom"]
    pool, o, err = _prefill(g, inp)
    assert err == 0
    print("oracle: T = 8192, 16 k-head groups in worker processes", flush=True)
    o_ref, finals, heads = OG.prefill_by_groups(g, inp)
    _check(g, inp, pool, o, heads=heads, ref=(o_ref, finals))


def test_workload4_varlen_one_head_per_group():
    """4 sequences, lengths uniform in [1024, 32768] (about 101 K tokens),
    nonzero initial states, long-memory gates; one v-head of every k-head
    group (each of the three positions in a group taken by some group)."""
    inp = gi.workload(4)
    g = inp["geom"]
    pool, o, err = _prefill(g, inp)
    assert err == 0
    G = g.n_v_heads // g.n_k_heads
    print("oracle: 101 K tokens, one v-head of each of the 16 k-head groups in worker processes", flush=True)
    o_ref, finals, heads = OG.prefill_by_groups(g, inp, heads_of_group=lambda kh: [kh * G + kh % G])
    _check(g, inp, pool, o, heads=heads, ref=(o_ref, finals))


def test_prefill_extreme_gates():
    """Gate inputs far out on both sides (a, b in {-40, -8, 0, 8, 40}, exact in
    bf16): alpha from 1 down to e^-40 and beta from e^-40 up to 1, so whole
    chunks decay to nothing and others carry the state unchanged."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=3)
    inp = gi.prefill_inputs(seed=560, geom=g, lengths=[200, 70], init_state=True)
    rng = np.random.Generator(np.random.PCG64(561))
    vals = np.array([-40.0, -8.0, 0.0, 8.0, 40.0], np.float32)
    inp["a"] = vals[rng.integers(0, 5, size=inp["a"].shape)]
    inp["b"] = vals[rng.integers(0, 5, size=inp["b"].shape)]
    # one stretch of long memory (alpha = 1, beta = 1) and one of full decay
    inp["a"][10:80] = -40.0
    inp["b"][10:80] = 40.0
    inp["a"][120:140] = 40.0
    pool, o, err = _prefill(g, inp)
    assert err == 0
    assert torch.isfinite(o.float()).all() and torch.isfinite(pool.state).all()
    _check(g, inp, pool, o)
