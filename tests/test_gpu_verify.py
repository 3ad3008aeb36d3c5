"""Speculative verify (k drafts, per-draft snapshots) and rollback on the GPU."""
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


def _verify(g, inp, pool, k):
    gdn = _gdn()
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    B = len(inp["slots"])
    snap = torch.empty(B, k, g.n_v_heads, g.d_v, g.d_k, dtype=torch.float32, device="cuda")
    o = torch.empty(B, k, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.verify_k(geom, pool, H.dev(inp["x"][:, :k], dt), H.dev(inp["a"][:, :k], dt), H.dev(inp["b"][:, :k], dt),
                 H.dev(inp["conv_w"]) if g.conv_width else None, H.dev(inp["slots"]), snap, o, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return snap, o


def test_verify_rollback_workload5():
    """4 slots x k = 4: snapshots and outputs vs the oracle; verify leaves the
    committed state and position alone; rollback to the seeded accepted lengths
    gives snap[a-1] bitwise and the oracle's replay of the accepted prefix."""
    gdn = _gdn()
    inp = gi.workload(5)
    g = inp["geom"]
    k = 4
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    state0 = pool.state.clone()
    pos0 = pool.conv_pos.clone()
    snap, o = _verify(g, inp, pool, k)
    assert torch.equal(pool.state, state0)
    assert torch.equal(pool.conv_pos, pos0)
    ref = []
    for i, s in enumerate(inp["slots"]):
        o_r, snaps_r, hists_r = orc.verify(g, inp["state"][s], inp["hist"][s], inp["x"][i], inp["a"][i],
                                           inp["b"][i], inp["conv_w"])
        assert H.relerr(H.f64(o[i]), o_r) <= H.TOL_BF16
        for j in range(k):
            assert H.relerr(snap[i, j].cpu().numpy(), snaps_r[j]) <= H.TOL_BF16, f"row {i} draft {j}"
        ref.append((snaps_r, hists_r))
    acc = inp["accepted"]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.rollback(H.to_geom(g), pool, snap, H.dev(inp["slots"]), H.dev(acc), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    hist = H.read_hist(g, pool)
    pos = H.positions(pool)
    for i, s in enumerate(inp["slots"]):
        n = int(acc[i])
        if n == 0:
            assert torch.equal(pool.state[s], state0[s])
        else:
            assert torch.equal(pool.state[s], snap[i, n - 1]), "rollback must be a bitwise copy"
        S_r, h_r = orc.rollback(inp["state"][s], inp["hist"][s], ref[i][0], ref[i][1], n)
        assert H.relerr(pool.state[s].cpu().numpy(), S_r) <= H.TOL_BF16
        assert np.array_equal(hist[s], h_r.astype(np.float32)), f"history after {n} accepted"
        assert pos[s] == inp["pos"][s] + n
    for s in range(g.n_slots):
        if s not in inp["slots"]:
            assert torch.equal(pool.state[s], state0[s])


@pytest.mark.parametrize("accepted", [[0, 1, 2, 3], [4, 4, 0, 2]])
def test_rollback_equals_decode_replay_bitwise(accepted):
    """The rolled-back state equals a GPU decode replay of the accepted drafts, bit for bit."""
    gdn = _gdn()
    inp = gi.workload(5, seed=9)
    g = inp["geom"]
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    snap, o = _verify(g, inp, pool, 4)
    acc = np.array(accepted, np.int32)
    gdn.rollback(geom, pool, snap, H.dev(inp["slots"]), H.dev(acc))
    replay = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    cw = H.dev(inp["conv_w"])
    for i, s in enumerate(inp["slots"]):
        for j in range(int(acc[i])):
            oj = torch.empty(1, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
            gdn.decode_step(geom, replay, H.dev(inp["x"][i:i + 1, j], dt), H.dev(inp["a"][i:i + 1, j], dt),
                            H.dev(inp["b"][i:i + 1, j], dt), cw, H.dev(np.array([s], np.int32)), oj)
            assert torch.equal(oj[0], o[i, j]), "verify output = decode output, bitwise"
    torch.cuda.synchronize()
    assert torch.equal(pool.state, replay.state)
    assert np.array_equal(H.read_hist(g, pool), H.read_hist(g, replay))
    assert np.array_equal(H.positions(pool), H.positions(replay))


def test_verify_k_smaller_than_max_and_fp32():
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=4, d_k=32, d_v=32, n_slots=3,
                            dtype_in=gi.F32, dtype_out=gi.F32, max_draft=4)
    inp = gi.decode_inputs(seed=41, geom=g, batch=2, n_tokens=2)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    snap, o = _verify(g, inp, pool, 2)
    for i, s in enumerate(inp["slots"]):
        o_r, snaps_r, _ = orc.verify(g, inp["state"][s], inp["hist"][s], inp["x"][i], inp["a"][i], inp["b"][i],
                                     inp["conv_w"])
        assert H.relerr(H.f64(o[i]), o_r) <= H.TOL_F32
        assert H.relerr(snap[i].cpu().numpy(), snaps_r) <= H.TOL_F32


def test_rollback_bad_accepted_reported():
    gdn = _gdn()
    inp = gi.workload(5, seed=3)
    g = inp["geom"]
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    snap, _ = _verify(g, inp, pool, 4)
    before = pool.state.clone()
    pos_before = pool.conv_pos.clone()
    acc = np.array([1, 7, -1, 0], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.rollback(H.to_geom(g), pool, snap, H.dev(inp["slots"]), H.dev(acc), dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gdn.DEV_BAD_ACCEPTED
    s0, s1, s2 = (int(s) for s in inp["slots"][:3])
    assert torch.equal(pool.state[s0], snap[0, 0])
    assert torch.equal(pool.state[s1], before[s1]) and torch.equal(pool.state[s2], before[s2])
    assert torch.equal(pool.conv_pos[s1], pos_before[s1]) and torch.equal(pool.conv_pos[s2], pos_before[s2])
