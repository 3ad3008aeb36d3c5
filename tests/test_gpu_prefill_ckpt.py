"""Prefill with state checkpoints at block boundaries, on the GPU, against the
fp64 oracle; and the checkpoints used the way prefix reuse uses them: a
second request resumes from one and continues exactly where the first left."""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import harness as H
from oracle import gdn_oracle as orc

pytestmark = pytest.mark.gpu


def _gdn():
    import gated_deltanet_delta_amd as gdn
    gdn.lib()
    return gdn


def _run(g, inp, every, pool=None):
    """Prefill with checkpoints every `every` tokens; returns (pool, o, ckpt, err)."""
    gdn = _gdn()
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    if pool is None:
        pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    N = inp["x"].shape[0]
    S = len(inp["cu_seqlens"]) - 1
    o = torch.zeros(N, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    ws = gdn.alloc_prefill_workspace(geom, N, S)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ckpt = torch.full((N // every, g.n_v_heads, g.d_v, g.d_k), float("nan"), device="cuda")
    gdn.prefill_chunked(geom, pool, H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt),
                        H.dev(inp["conv_w"]) if g.conv_width else None, H.dev(inp["cu_seqlens"]),
                        H.dev(inp["slots"]), H.dev(inp["has_init"]), o, ws, dev_err=err,
                        ckpt=ckpt, ckpt_every=every)
    torch.cuda.synchronize()
    return pool, o, ckpt, int(err.item())


def _plain(g, inp):
    gdn = _gdn()
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    N = inp["x"].shape[0]
    S = len(inp["cu_seqlens"]) - 1
    o = torch.zeros(N, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    ws = gdn.alloc_prefill_workspace(geom, N, S)
    gdn.prefill_chunked(geom, pool, H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt),
                        H.dev(inp["conv_w"]) if g.conv_width else None, H.dev(inp["cu_seqlens"]),
                        H.dev(inp["slots"]), H.dev(inp["has_init"]), o, ws)
    torch.cuda.synchronize()
    return pool, o


def _check_ckpts(g, inp, every, ckpt, heads=None):
    heads_l = list(range(g.n_v_heads)) if heads is None else list(heads)
    S = len(inp["cu_seqlens"]) - 1
    S0 = np.stack([inp["state"][s] for s in inp["slots"]])
    h0 = np.stack([inp["hist"][s] for s in inp["slots"]]) if g.conv_width else np.zeros((S, 0, g.conv_channels))
    _, _, ck_ref, where = orc.prefill_checkpoints(g, inp["x"], inp["a"], inp["b"], inp["conv_w"],
                                                  inp["cu_seqlens"], S0, h0, inp["has_init"], every, heads=heads)
    lens = np.diff(inp["cu_seqlens"])
    n = _gdn().checkpoint_count(lens, every)
    assert n == len(where)
    got = ckpt.cpu().numpy()
    tol = H.tol_for(g)
    for i, (s, p) in enumerate(where):
        e = H.relerr(got[i][heads_l], ck_ref[i])
        assert e <= tol, f"checkpoint {i} (seq {s}, after {p} tokens) rel err {e:.3e}"
    # entries past the last checkpoint are not touched
    assert torch.isnan(ckpt[n:]).all()
    return where


def _same_as_plain(g, inp, pool, o):
    """Everything the plain prefill writes is written bit for bit the same."""
    pool0, o0 = _plain(g, inp)
    assert torch.equal(o, o0)
    assert torch.equal(pool.state, pool0.state)
    assert torch.equal(pool.conv_state, pool0.conv_state)
    assert torch.equal(pool.conv_pos, pool0.conv_pos)


@pytest.mark.parametrize("every", [64, 128, 320])
def test_checkpoints_varlen_bf16(every):
    """Lengths 300, 0, 640, 129 (an empty sequence, one that ends on a block
    boundary, partial last chunks), with and without initial state."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=5)
    inp = gi.prefill_inputs(seed=600 + every, geom=g, lengths=[300, 0, 640, 129], a_mean=-2.0)
    inp["has_init"] = np.array([1, 1, 0, 1], np.int32)
    pool, o, ckpt, err = _run(g, inp, every)
    assert err == 0
    where = _check_ckpts(g, inp, every, ckpt)
    assert (2, 640) in where or 640 % every
    _same_as_plain(g, inp, pool, o)
    # a sequence that ends on a boundary: its last checkpoint is its final state
    if 640 % every == 0:
        i = where.index((2, 640))
        assert torch.equal(ckpt[i], pool.state[int(inp["slots"][2])])


@pytest.mark.parametrize("every", [528, 100, 40, 7])
def test_checkpoints_inside_chunks_bf16(every):
    """Blocks that end inside a chunk ([Hybrid] section 4.2's 528-token block,
    and blocks shorter than a chunk, several per chunk): lengths 1100, 0, 530
    and 64 with and without initial state."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=5)
    inp = gi.prefill_inputs(seed=620 + every, geom=g, lengths=[1100, 0, 530, 64], a_mean=-2.0)
    inp["has_init"] = np.array([1, 0, 0, 1], np.int32)
    pool, o, ckpt, err = _run(g, inp, every)
    assert err == 0
    _check_ckpts(g, inp, every, ckpt)
    _same_as_plain(g, inp, pool, o)


def test_checkpoints_fp32():
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=3, d_k=32, d_v=32, n_slots=4,
                            dtype_in=gi.F32, dtype_out=gi.F32)
    inp = gi.prefill_inputs(seed=610, geom=g, lengths=[70, 257, 128], init_state=True)
    for every in (64, 45):
        pool, o, ckpt, err = _run(g, inp, every)
        assert err == 0
        _check_ckpts(g, inp, every, ckpt)
        _same_as_plain(g, inp, pool, o)


@pytest.mark.parametrize("every", [512, 528])
def test_checkpoints_full_geometry_all_heads(every):
    """48 v-heads at d = 128, 1100 tokens, a checkpoint every 512 tokens (on
    chunk ends) or every 528 (the hybrid model's cache block, inside chunks);
    every head of every checkpoint against the oracle."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=2)
    inp = gi.prefill_inputs(seed=611, geom=g, lengths=[1100], init_state=True, a_mean=-2.0)
    pool, o, ckpt, err = _run(g, inp, every)
    assert err == 0
    _check_ckpts(g, inp, every, ckpt)
    _same_as_plain(g, inp, pool, o)


@pytest.mark.parametrize("lengths", [[600, 70], [300, 400]])
def test_checkpoints_segmented_launches(lengths):
    """32 k-heads x 8 v-heads: two launches over k-head ranges; checkpoints
    every 256 tokens in both sequences (the second sequence's numbered after
    the first's), heads on both sides of the split."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=32, n_v_heads=256, n_slots=2)
    inp = gi.prefill_inputs(seed=612 + lengths[1], geom=g, lengths=lengths, init_state=True, a_mean=-2.0)
    pool, o, ckpt, err = _run(g, inp, 256)
    assert err == 0
    _check_ckpts(g, inp, 256, ckpt, heads=[0, 191, 192, 255])


def test_resume_from_a_checkpoint_continues_the_request():
    """Prefix reuse: request 1 (p + 200 tokens) writes a checkpoint after p
    tokens; request 2 starts from that checkpoint and the conv history x rows
    p-3 .. p-1 in a fresh slot and prefills the same 200 tokens.  Its outputs
    and final state equal request 1's bit for bit."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=3)
    p, tail, every = 384, 200, 128
    inp = gi.prefill_inputs(seed=613, geom=g, lengths=[p + tail], init_state=True, a_mean=-2.0)
    pool1, o1, ckpt, err = _run(g, inp, every)
    assert err == 0
    slot1 = int(inp["slots"][0])
    slot2 = next(s for s in range(g.n_slots) if s != slot1)
    # the resumed slot: checkpoint p / every - 1, history = the inputs before p
    state = np.array(inp["state"])
    state[slot2] = ckpt[p // every - 1].cpu().numpy()
    hist = np.array(inp["hist"])
    hist[slot2] = inp["x"][p - (g.conv_width - 1):p].astype(np.float32)
    pos = np.array(inp["pos"])
    pos[slot2] = 7 * p + 3  # any ring position: only the history rows matter
    inp2 = dict(inp, x=inp["x"][p:], a=inp["a"][p:], b=inp["b"][p:],
                cu_seqlens=np.array([0, tail], np.int32), slots=np.array([slot2], np.int32),
                has_init=np.array([1], np.int32), state=state, hist=hist, pos=pos)
    pool2, o2, _, err = _run(g, inp2, every)
    assert err == 0
    assert torch.equal(o2, o1[p:])
    assert torch.equal(pool2.state[slot2], pool1.state[slot1])
    assert np.array_equal(H.read_hist(g, pool2)[slot2], H.read_hist(g, pool1)[slot1])
    assert gdn.checkpoint_count([tail], every) == 1


@pytest.mark.parametrize("lengths", [[0, 5], [0, 0]])
def test_checkpoints_none_due(lengths):
    """Sequences shorter than a block (and no tokens at all): no checkpoint is
    written, an empty checkpoint buffer is accepted, and everything else is
    what the plain prefill writes."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=3)
    inp = gi.prefill_inputs(seed=620 + sum(lengths), geom=g, lengths=lengths, init_state=True)
    inp["has_init"] = np.array([0, 1], np.int32)
    pool, o, ckpt, err = _run(g, inp, 64)
    assert err == 0
    assert ckpt.shape[0] == 0
    _same_as_plain(g, inp, pool, o)
