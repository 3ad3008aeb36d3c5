"""Verify into pool slots and zero-copy commit, on the GPU: every snapshot is
a whole slot (state, conv history, position); the commit only picks a slot
id.  Checked against the oracle and bit for bit against verify + rollback."""
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


def _snap_slots(g, slots, k):
    """Distinct pool slots for the snapshots: the ones no row uses, in order."""
    free = [s for s in range(g.n_slots) if s not in set(int(x) for x in slots)]
    assert len(free) >= len(slots) * k
    return np.array(free[:len(slots) * k], np.int32).reshape(len(slots), k)


def _run_both(g, inp, k, accepted):
    """The copy path (verify + rollback) on one pool, the slot path (verify
    into slots + commit) on an identical pool."""
    gdn = _gdn()
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    B = len(inp["slots"])
    x, a, b = (H.dev(inp[n][:, :k], dt) for n in ("x", "a", "b"))
    cw = H.dev(inp["conv_w"])
    slot = H.dev(inp["slots"])
    acc = H.dev(np.asarray(accepted, np.int32))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    snap = torch.empty(B, k, g.n_v_heads, g.d_v, g.d_k, dtype=torch.float32, device="cuda")
    oa = torch.empty(B, k, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    gdn.verify_k(geom, pa, x, a, b, cw, slot, snap, oa, dev_err=err)
    gdn.rollback(geom, pa, snap, slot, acc, dev_err=err)
    pb = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    ss = _snap_slots(g, inp["slots"], k)
    ob = torch.empty_like(oa)
    nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    gdn.verify_k_slots(geom, pb, x, a, b, cw, slot, H.dev(ss), ob, dev_err=err)
    gdn.commit_slots(geom, slot, H.dev(ss), acc, nxt, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return pa, snap, oa, pb, ss, ob, nxt


def test_verify_slots_equals_the_copy_path():
    """4 rows x k = 4 with accepted 0..4: outputs, every snapshot slot, and the
    committed slot's state, history and position equal verify + rollback bit
    for bit, and the oracle within 2e-2; a decode step then continues both
    paths identically."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=24)
    inp = gi.verify_inputs(seed=710, geom=g, batch=4, k=4)
    k = 4
    accepted = [0, 1, 4, 2]
    pa, snap, oa, pb, ss, ob, nxt = _run_both(g, inp, k, accepted)
    assert torch.equal(oa, ob)
    hist_b = H.read_hist(g, pb)
    pos_b = H.positions(pb)
    for i, s in enumerate(inp["slots"]):
        p0 = int(inp["pos"][s])
        o_r, snaps_r, hists_r = orc.verify(g, inp["state"][s], inp["hist"][s], inp["x"][i, :k], inp["a"][i, :k],
                                           inp["b"][i, :k], inp["conv_w"])
        for j in range(k):
            sj = int(ss[i, j])
            assert torch.equal(pb.state[sj], snap[i, j]), f"row {i} snapshot {j} differs from verify_k's"
            assert H.relerr(pb.state[sj].cpu().numpy(), snaps_r[j]) <= H.TOL_BF16
            assert np.array_equal(hist_b[sj], hists_r[j].astype(np.float32)), f"row {i} snapshot {j} history"
            assert pos_b[sj] == p0 + j + 1
        # the row's own slot keeps its state and position
        assert torch.equal(pb.state[s], torch.from_numpy(inp["state"][s]).cuda())
        assert pos_b[s] == p0
    nxt_h = nxt.cpu().numpy()
    hist_a = H.read_hist(g, pa)
    pos_a = H.positions(pa)
    for i, s in enumerate(inp["slots"]):
        n = accepted[i]
        want = int(s) if n == 0 else int(ss[i, n - 1])
        assert nxt_h[i] == want
        assert torch.equal(pb.state[want], pa.state[s])
        assert np.array_equal(hist_b[want], hist_a[s])
        assert pos_b[want] == pos_a[s]
    # one more token through both: bit-identical outputs and states
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    rng = np.random.Generator(np.random.PCG64(711))
    dx = H.dev(rng.normal(size=(4, g.conv_channels)).astype(np.float32), dt)
    da = H.dev(rng.normal(size=(4, g.n_v_heads)).astype(np.float32), dt)
    db = H.dev(rng.normal(size=(4, g.n_v_heads)).astype(np.float32), dt)
    cw = H.dev(inp["conv_w"])
    o1 = torch.empty(4, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    o2 = torch.empty_like(o1)
    gdn.decode_step(geom, pa, dx, da, db, cw, H.dev(inp["slots"]), o1)
    gdn.decode_step(geom, pb, dx, da, db, cw, nxt, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for i, s in enumerate(inp["slots"]):
        assert torch.equal(pa.state[s], pb.state[int(nxt_h[i])])


@pytest.mark.parametrize("accepted", [[1, 5, 3], [5, 1, 2]])
def test_verify_slots_k_plus_one_rows(accepted):
    """The last accepted token verified with its 4 drafts as k + 1 = 5 rows
    (max_draft 5): at least the first row is always accepted; the committed
    slot holds the oracle's state and history after those rows."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=4, n_v_heads=12, n_slots=20, max_draft=5)
    k = 5
    inp = gi.verify_inputs(seed=720 + accepted[0], geom=g, batch=3, k=k)
    pa, snap, oa, pb, ss, ob, nxt = _run_both(g, inp, k, accepted)
    hist_b = H.read_hist(g, pb)
    pos_b = H.positions(pb)
    nxt_h = nxt.cpu().numpy()
    for i, s in enumerate(inp["slots"]):
        o_r, snaps_r, hists_r = orc.verify(g, inp["state"][s], inp["hist"][s], inp["x"][i], inp["a"][i],
                                           inp["b"][i], inp["conv_w"])
        assert H.relerr(H.f64(ob[i]), o_r) <= H.TOL_BF16
        n = accepted[i]
        S_r, h_r = orc.rollback(inp["state"][s], inp["hist"][s], snaps_r, hists_r, n)
        t = int(nxt_h[i])
        assert t == int(ss[i, n - 1])
        assert H.relerr(pb.state[t].cpu().numpy(), S_r) <= H.TOL_BF16
        assert np.array_equal(hist_b[t], h_r.astype(np.float32))
        assert pos_b[t] == int(inp["pos"][s]) + n
        assert torch.equal(pb.state[t], pa.state[s])


def test_verify_slots_bad_ids_reported():
    """A snapshot slot id out of range sets GDN_DEV_BAD_SLOT and only that
    snapshot is skipped; an accepted length out of range sets
    GDN_DEV_BAD_ACCEPTED and keeps the row's own slot."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=12)
    k = 2
    inp = gi.verify_inputs(seed=730, geom=g, batch=2, k=k)
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    ss = _snap_slots(g, inp["slots"], k)
    good = int(ss[1, 1])
    ss[0, 1] = g.n_slots + 7
    before = pool.state.clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty(2, k, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    gdn.verify_k_slots(geom, pool, *(H.dev(inp[n][:, :k], dt) for n in ("x", "a", "b")), H.dev(inp["conv_w"]),
                       H.dev(inp["slots"]), H.dev(ss), o, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gdn.DEV_BAD_SLOT
    assert not torch.equal(pool.state[good], before[good])  # the valid snapshots were written
    err.zero_()
    nxt = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    gdn.commit_slots(geom, H.dev(inp["slots"]), H.dev(ss), H.dev(np.array([k + 1, 1], np.int32)), nxt, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gdn.DEV_BAD_ACCEPTED
    assert nxt.cpu().tolist() == [int(inp["slots"][0]), int(ss[1, 0])]


def test_verify_slots_per_row_k():
    """Rows verify 4, 1, 3 and 2 drafts in one call: each row's snapshots equal
    a call of its own with that k, bit for bit, and the oracle within 2e-2;
    nothing past a row's count is written; the commit picks within each
    row's count; a count of 0 sets GDN_DEV_BAD_K."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=4, n_v_heads=12, n_slots=24)
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    k, kr, acc = 4, [4, 1, 3, 2], [3, 1, 0, 2]
    inp = gi.verify_inputs(seed=740, geom=g, batch=4, k=k)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    state0 = pool.state.clone()
    ss = _snap_slots(g, inp["slots"], k)
    x, a, b = (H.dev(inp[n], dt) for n in ("x", "a", "b"))
    cw = H.dev(inp["conv_w"])
    o = torch.full((4, k, g.n_v_heads, g.d_v), float("nan"), dtype=dt, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    nxt = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    gdn.verify_k_slots(geom, pool, x, a, b, cw, H.dev(inp["slots"]), H.dev(ss), o, dev_err=err,
                       k_row=H.dev(np.array(kr, np.int32)))
    gdn.commit_slots(geom, H.dev(inp["slots"]), H.dev(ss), H.dev(np.array(acc, np.int32)), nxt, dev_err=err,
                     k_row=H.dev(np.array(kr, np.int32)))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    hist = H.read_hist(g, pool)
    pos = H.positions(pool)
    for i, s in enumerate(inp["slots"]):
        n = kr[i]
        o_r, snaps_r, hists_r = orc.verify(g, inp["state"][s], inp["hist"][s], inp["x"][i, :n], inp["a"][i, :n],
                                           inp["b"][i, :n], inp["conv_w"])
        assert H.relerr(H.f64(o[i, :n]), o_r) <= H.TOL_BF16
        assert torch.isnan(o[i, n:].float()).all(), f"row {i}: outputs past its count were written"
        # the row alone, with its own k, in a pool of its own
        alone = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
        oa = torch.empty(1, n, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
        gdn.verify_k_slots(geom, alone, x[i:i + 1, :n].contiguous(), a[i:i + 1, :n].contiguous(),
                           b[i:i + 1, :n].contiguous(), cw, H.dev(inp["slots"][i:i + 1]),
                           H.dev(np.ascontiguousarray(ss[i:i + 1, :n])), oa, dev_err=err)
        torch.cuda.synchronize()
        assert torch.equal(oa[0], o[i, :n])
        for j in range(k):
            sj = int(ss[i, j])
            if j < n:
                assert torch.equal(pool.state[sj], alone.state[sj])
                assert H.relerr(pool.state[sj].cpu().numpy(), snaps_r[j]) <= H.TOL_BF16
                assert np.array_equal(hist[sj], hists_r[j].astype(np.float32))
                assert pos[sj] == int(inp["pos"][s]) + j + 1
            else:
                assert torch.equal(pool.state[sj], state0[sj]), f"row {i}: snapshot slot {j} past its count"
        want = int(s) if acc[i] == 0 else int(ss[i, acc[i] - 1])
        assert int(nxt[i].item()) == want
    # a count out of range: reported, that row skipped
    err.zero_()
    before = pool.state.clone()
    bad = np.array([0, 1, 1, 1], np.int32)
    gdn.verify_k_slots(geom, pool, x, a, b, cw, H.dev(inp["slots"]), H.dev(ss), o, dev_err=err, k_row=H.dev(bad))
    torch.cuda.synchronize()
    assert int(err.item()) == gdn.DEV_BAD_K
    assert torch.equal(pool.state[int(ss[0, 0])], before[int(ss[0, 0])])


@pytest.mark.parametrize("conv_width,dtype", [(0, gi.BF16), (4, gi.F32)])
def test_verify_slots_other_geometries(conv_width, dtype):
    """No conv front end (snapshot slots get the state only), and fp32
    inputs at d = 32: the slot path equals verify + rollback bit for bit."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, d_k=32, d_v=32, n_slots=16,
                            conv_width=conv_width, dtype_in=dtype, dtype_out=dtype, l2norm_qk=conv_width > 0)
    k = 3
    inp = gi.verify_inputs(seed=750 + conv_width, geom=g, batch=3, k=k)
    accepted = [2, 0, 3]
    pa, snap, oa, pb, ss, ob, nxt = _run_both(g, inp, k, accepted)
    assert torch.equal(oa, ob)
    nxt_h = nxt.cpu().numpy()
    for i, s in enumerate(inp["slots"]):
        for j in range(k):
            assert torch.equal(pb.state[int(ss[i, j])], snap[i, j])
        assert torch.equal(pb.state[int(nxt_h[i])], pa.state[s])
        o_r, snaps_r, hists_r = orc.verify(g, inp["state"][s], inp["hist"][s], inp["x"][i], inp["a"][i],
                                           inp["b"][i], inp["conv_w"])
        assert H.relerr(H.f64(ob[i]), o_r) <= H.tol_for(g)
    if conv_width:
        hist_a, hist_b = H.read_hist(g, pa), H.read_hist(g, pb)
        for i, s in enumerate(inp["slots"]):
            assert np.array_equal(hist_b[int(nxt_h[i])], hist_a[s])
