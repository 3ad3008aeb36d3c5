"""Decode, verify, rollback and the chunked prefill captured in a HIP graph:
every replay, with eager work and synchronisations between the replays, gives
the eager results bit for bit (the token-path calls launch kernels only, on
the caller's stream, so they can be captured; a serving loop replays them),
and the eager results of the layer stack match the fp64 oracle."""
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


def _pool_copy(pool):
    return [t.clone() for t in (pool.state, pool.conv_state, pool.conv_pos)]


def _pool_set(pool, saved):
    for t, s in zip((pool.state, pool.conv_state, pool.conv_pos), saved):
        t.copy_(s)


def test_graph_replays_match_eager():
    gdn = _gdn()
    d_inp = gi.workload(2)
    v_inp = gi.workload(5)
    g = d_inp["geom"]
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    k = 4
    B = len(d_inp["slots"])
    dpool = H.make_pool(g, d_inp["state"], d_inp["hist"], d_inp["pos"])
    vpool = H.make_pool(g, v_inp["state"], v_inp["hist"], v_inp["pos"])
    d0, v0 = _pool_copy(dpool), _pool_copy(vpool)
    cw = H.dev(d_inp["conv_w"])
    dx, da, db = (H.dev(d_inp[n][:, 0], dt) for n in ("x", "a", "b"))
    vx, va, vb = (H.dev(v_inp[n][:, :k], dt) for n in ("x", "a", "b"))
    dslot, vslot, vacc = H.dev(d_inp["slots"]), H.dev(v_inp["slots"]), H.dev(v_inp["accepted"])
    do = torch.empty(B, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    vo = torch.empty(B, k, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    snap = torch.empty(B, k, g.n_v_heads, g.d_v, g.d_k, dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def calls():
        gdn.decode_step(geom, dpool, dx, da, db, cw, dslot, do, dev_err=err)
        gdn.verify_k(geom, vpool, vx, va, vb, cw, vslot, snap, vo, dev_err=err)
        gdn.rollback(geom, vpool, snap, vslot, vacc, dev_err=err)

    def results():
        return [t.clone() for t in (do, vo, snap, *_pool_copy(dpool), *_pool_copy(vpool))]

    # eager reference
    calls()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = results()

    # warm-up on a side stream, then capture
    _pool_set(dpool, d0)
    _pool_set(vpool, v0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between the replays: reset the pools, clobber the outputs
        _pool_set(dpool, d0)
        _pool_set(vpool, v0)
        for t in (do, vo, snap):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        got = results()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: result {i} differs from the eager run"


def test_layer_stack_graph_replays_match_eager():
    """Three layers, each with its own slot pool, conv weights and inputs: one
    graph holds a decode token and a verify + rollback round through all of
    them; every replay gives the eager results bit for bit."""
    gdn = _gdn()
    n_layers = 3
    layers = [(gi.workload(2, seed=70 + l), gi.workload(5, seed=80 + l)) for l in range(n_layers)]
    g = layers[0][0]["geom"]
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    k = 4
    B = len(layers[0][0]["slots"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pools, saved, args = [], [], []
    for d_inp, v_inp in layers:
        pool = H.make_pool(g, d_inp["state"], d_inp["hist"], d_inp["pos"])
        pools.append(pool)
        saved.append(_pool_copy(pool))
        args.append(dict(
            cw=H.dev(d_inp["conv_w"]),
            dx=H.dev(d_inp["x"][:, 0], dt), da=H.dev(d_inp["a"][:, 0], dt), db=H.dev(d_inp["b"][:, 0], dt),
            vx=H.dev(v_inp["x"][:, :k], dt), va=H.dev(v_inp["a"][:, :k], dt), vb=H.dev(v_inp["b"][:, :k], dt),
            dslot=H.dev(d_inp["slots"]), vslot=H.dev(v_inp["slots"]), vacc=H.dev(v_inp["accepted"]),
            do=torch.empty(B, g.n_v_heads, g.d_v, dtype=dt, device="cuda"),
            vo=torch.empty(B, k, g.n_v_heads, g.d_v, dtype=dt, device="cuda"),
            snap=torch.empty(B, k, g.n_v_heads, g.d_v, g.d_k, dtype=torch.float32, device="cuda")))

    def calls():
        for pool, a in zip(pools, args):
            gdn.decode_step(geom, pool, a["dx"], a["da"], a["db"], a["cw"], a["dslot"], a["do"], dev_err=err)
            gdn.verify_k(geom, pool, a["vx"], a["va"], a["vb"], a["cw"], a["vslot"], a["snap"], a["vo"],
                         dev_err=err)
            gdn.rollback(geom, pool, a["snap"], a["vslot"], a["vacc"], dev_err=err)

    def reset():
        for pool, s in zip(pools, saved):
            _pool_set(pool, s)

    def results():
        out = []
        for pool, a in zip(pools, args):
            out += [a["do"].clone(), a["vo"].clone(), a["snap"].clone(), *_pool_copy(pool)]
        return out

    calls()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = results()
    # the eager results (which every replay must equal bit for bit) against
    # the oracle: per layer, the decode token, then verify of k drafts from
    # the state the decode left, then rollback to the accepted drafts
    for l, ((d_inp, v_inp), a) in enumerate(zip(layers, args)):
        st, hi = np.array(d_inp["state"], np.float64), np.array(d_inp["hist"], np.float64)
        do_r, st, hi = orc.decode_step(g, st, hi, d_inp["x"][:, 0], d_inp["a"][:, 0], d_inp["b"][:, 0],
                                       d_inp["conv_w"], d_inp["slots"])
        assert H.relerr(H.f64(a["do"]), do_r) <= H.TOL_BF16, f"layer {l}: decode output"
        for i, s in enumerate(v_inp["slots"]):
            o_r, snaps_r, hists_r = orc.verify(g, st[s], hi[s], v_inp["x"][i, :k], v_inp["a"][i, :k],
                                               v_inp["b"][i, :k], d_inp["conv_w"])
            assert H.relerr(H.f64(a["vo"][i]), o_r) <= H.TOL_BF16, f"layer {l} row {i}: verify outputs"
            assert H.relerr(a["snap"][i].cpu().numpy(), snaps_r) <= H.TOL_BF16, f"layer {l} row {i}: snapshots"
            S_r, h_r = orc.rollback(st[s], hi[s], snaps_r, hists_r, int(v_inp["accepted"][i]))
            st[s], hi[s] = S_r, h_r
        assert H.relerr(pools[l].state.cpu().numpy(), st) <= H.TOL_BF16, f"layer {l}: states after the round"
        assert np.array_equal(H.read_hist(g, pools[l]), hi.astype(np.float32)), f"layer {l}: conv histories"
    reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        for a in args:
            for t in (a["do"], a["vo"], a["snap"]):
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for i, (x, y) in enumerate(zip(results(), ref)):
            assert torch.equal(x, y), f"replay {rep}: result {i} differs from the eager run"


def test_prefill_graph_replays_match_eager():
    """A varlen chunked prefill with checkpoints (lengths 700, 0, 333, 1: an
    empty sequence, partial chunks, mixed initial states, blocks ending inside
    chunks), the same prefill through the static workspace, then a decode
    token on the prefilled slots, all in one graph: every replay, with the pools
    reset and the outputs clobbered eagerly between replays, equals the eager
    run bit for bit; the eager prefill matches the oracle."""
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=6)
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    inp = gi.prefill_inputs(seed=950, geom=g, lengths=[700, 0, 333, 1], init_state=True, a_mean=-2.0)
    inp["has_init"] = np.array([1, 1, 0, 1], np.int32)
    N = inp["x"].shape[0]
    S = len(inp["cu_seqlens"]) - 1
    every = 300
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    pool2 = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    saved, saved2 = _pool_copy(pool), _pool_copy(pool2)
    args = (H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt), H.dev(inp["conv_w"]),
            H.dev(inp["cu_seqlens"]), H.dev(inp["slots"]), H.dev(inp["has_init"]))
    o = torch.empty(N, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    o2 = torch.empty_like(o)
    ckpt = torch.empty(N // every, g.n_v_heads, g.d_v, g.d_k, dtype=torch.float32, device="cuda")
    ws = gdn.alloc_prefill_workspace(geom, N, S)
    rng = np.random.default_rng(951)
    dx = H.dev(rng.standard_normal((S, g.conv_channels)).astype(np.float32), dt)
    da = H.dev(rng.standard_normal((S, g.n_v_heads)).astype(np.float32), dt)
    db = H.dev(rng.standard_normal((S, g.n_v_heads)).astype(np.float32), dt)
    do = torch.empty(S, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def calls():
        gdn.prefill_chunked(geom, pool, *args, o, ws, dev_err=err, ckpt=ckpt, ckpt_every=every)
        gdn.prefill_chunked_static(geom, pool2, *args, o2, dev_err=err)
        gdn.decode_step(geom, pool, dx, da, db, args[3], args[5], do, dev_err=err)

    def reset():
        _pool_set(pool, saved)
        _pool_set(pool2, saved2)
        for t in (o, o2, ckpt, do):
            t.fill_(float("nan"))

    def results():
        return [t.clone() for t in (o, o2, ckpt, do, *_pool_copy(pool), *_pool_copy(pool2))]

    reset()
    calls()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = results()
    assert torch.equal(ref[0], ref[1]), "static-workspace prefill differs from the prefill"
    S0 = np.stack([inp["state"][s] for s in inp["slots"]])
    h0 = np.stack([inp["hist"][s] for s in inp["slots"]])
    o_r, finals = orc.prefill(g, inp["x"], inp["a"], inp["b"], inp["conv_w"], inp["cu_seqlens"], S0, h0,
                              inp["has_init"])
    assert H.relerr(H.f64(ref[0]), o_r) <= H.TOL_BF16
    state2 = ref[7].cpu().numpy()  # the static-workspace pool: the prefill's final states, no decode after
    for s, (S_T, _) in enumerate(finals):
        assert H.relerr(state2[int(inp["slots"][s])], S_T) <= H.TOL_BF16, f"seq {s} final state"
    reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        # eager work of the program's own between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for i, (x, y) in enumerate(zip(results(), ref)):
            assert torch.equal(x, y), f"replay {rep}: result {i} differs from the eager run"
        del scratch
