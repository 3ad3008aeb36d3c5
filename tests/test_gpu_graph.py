"""Decode, verify and rollback captured in a HIP graph: every replay, with
eager work and synchronisations between the replays, gives the eager results
bit for bit (the token-path calls launch kernels only, so they can be
captured; a serving loop replays them)."""
import pytest
import torch

import gdn_inputs as gi
import harness as H

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
