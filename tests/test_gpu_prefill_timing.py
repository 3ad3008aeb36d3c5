"""Kernel-timing events of the prefill (gdn_prefill_timing_events): the events
are recorded by the call's kernel launches and bracket them (positive, no
longer than the call timed by stream events, outputs unchanged bit for bit), the
request is consumed by one call, and a pending request under graph capture is
refused before anything is launched or captured."""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import harness as H

pytestmark = pytest.mark.gpu


def _setup(T=2048, seed=960):
    import gated_deltanet_delta_amd as gdn
    gdn.lib()
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=2)
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    inp = gi.prefill_inputs(seed=seed, geom=g, lengths=[T], init_state=True)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    args = (H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt), H.dev(inp["conv_w"]),
            H.dev(inp["cu_seqlens"]), H.dev(inp["slots"]), H.dev(inp["has_init"]))
    o = torch.empty(T, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    ws = gdn.alloc_prefill_workspace(geom, T, 1)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    saved = [t.clone() for t in (pool.state, pool.conv_state, pool.conv_pos)]

    def reset():
        for t, s in zip((pool.state, pool.conv_state, pool.conv_pos), saved):
            t.copy_(s)

    def call():
        gdn.prefill_chunked(geom, pool, *args, o, ws, dev_err=err)

    def results():
        return [t.clone() for t in (o, pool.state, pool.conv_state, pool.conv_pos)]

    return gdn, reset, call, results, err


def _events():
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()  # the HIP events exist from here on
    torch.cuda.synchronize()
    return e0, e1


def test_kernel_events_bracket_the_kernel():
    gdn, reset, call, results, err = _setup()
    reset()
    call()
    torch.cuda.synchronize()
    ref = results()
    k0, k1 = _events()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for rep in range(3):
        reset()
        gdn.prefill_timing_events(k0, k1)
        call()
        torch.cuda.synchronize()
        t_kernel = k0.elapsed_time(k1)
        reset()
        s0.record()
        call()  # the request was consumed: a plain call
        s1.record()
        torch.cuda.synchronize()
        t_call = s0.elapsed_time(s1)
        assert int(err.item()) == 0
        for i, (a, b) in enumerate(zip(results(), ref)):
            assert torch.equal(a, b), f"rep {rep}: result {i} differs"
        assert 0.0 < t_kernel <= t_call * 1.02 + 0.005, (t_kernel, t_call)


def test_pending_request_refused_under_capture():
    gdn, reset, call, results, err = _setup(T=300, seed=961)
    reset()
    call()
    torch.cuda.synchronize()
    ref = results()
    k0, k1 = _events()
    reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.prefill_timing_events(k0, k1)
        with pytest.raises(gdn.GdnError) as info:
            call()
        call()  # consumed by the refused call: this one is captured
    assert info.value.status == 7 and "HIP launch failed" in info.value.message
    torch.cuda.synchronize()
    for rep in range(2):
        reset()
        o_junk = torch.randn(1 << 18, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for i, (a, b) in enumerate(zip(results(), ref)):
            assert torch.equal(a, b), f"replay {rep}: result {i} differs from the eager run"
        del o_junk


def test_every_prefill_entry_point_takes_the_request():
    """The static-workspace prefill and the prefill with checkpoints record the
    events too (each consumes the request), with results unchanged."""
    import gated_deltanet_delta_amd as gdn
    gdn.lib()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=2)
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    T, every = 700, 256
    inp = gi.prefill_inputs(seed=962, geom=g, lengths=[T], init_state=True)
    args = (H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt), H.dev(inp["conv_w"]),
            H.dev(inp["cu_seqlens"]), H.dev(inp["slots"]), H.dev(inp["has_init"]))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = gdn.alloc_prefill_workspace(geom, T, 1)
    k0, k1 = _events()

    def run(kind, timed):
        pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
        o = torch.empty(T, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
        ckpt = torch.empty(T // every, g.n_v_heads, g.d_v, g.d_k, dtype=torch.float32, device="cuda")
        if timed:
            gdn.prefill_timing_events(k0, k1)
        if kind == "static":
            gdn.prefill_chunked_static(geom, pool, *args, o, dev_err=err)
        else:
            gdn.prefill_chunked(geom, pool, *args, o, ws, dev_err=err, ckpt=ckpt, ckpt_every=every)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        return [o, pool.state, pool.conv_state, pool.conv_pos] + ([ckpt] if kind == "ckpt" else [])

    for kind in ("static", "ckpt"):
        ref = run(kind, False)
        got = run(kind, True)
        assert k0.elapsed_time(k1) > 0.0, kind
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"{kind}: result {i} differs with timing events"
