"""The prefill that allocates nothing (the library's static workspace) against
the prefill with a workspace of the caller's: the same kernels, so every
output, state, conv history and position must agree bit for bit.  Two calls
in a row share the static workspace, the second with a smaller input, so the
second must not see anything the first left there."""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
import harness as H

pytestmark = pytest.mark.gpu


def _gdn():
    import gated_deltanet_delta_amd as gdn
    gdn.lib()
    return gdn


def _both(g, inp):
    """Run both entry points from the same slot pool; returns their results."""
    gdn = _gdn()
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    N = inp["x"].shape[0]
    S = len(inp["cu_seqlens"]) - 1
    args = (H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt),
            H.dev(inp["conv_w"]) if g.conv_width else None, H.dev(inp["cu_seqlens"]),
            H.dev(inp["slots"]), H.dev(inp["has_init"]))
    out = []
    for static in (False, True):
        pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
        o = torch.full((N, g.n_v_heads, g.d_v), float("nan"), dtype=dt, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if static:
            gdn.prefill_chunked_static(geom, pool, *args, o, dev_err=err)
        else:
            ws = gdn.alloc_prefill_workspace(geom, N, S)
            gdn.prefill_chunked(geom, pool, *args, o, ws, dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, f"static={static}: device error {int(err.item())}"
        out.append((o, pool))
    return out


def _same(a, b):
    (o1, p1), (o2, p2) = a, b
    assert torch.equal(o1, o2)
    assert torch.equal(p1.state, p2.state)
    assert torch.equal(p1.conv_state, p2.conv_state)
    assert torch.equal(p1.conv_pos, p2.conv_pos)


def test_static_workspace_matches_caller_workspace_two_calls():
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=4)
    print("static-workspace prefill: call 1, lengths [700, 0, 333, 64], 48 v-heads", flush=True)
    inp = gi.prefill_inputs(seed=901, geom=g, lengths=[700, 0, 333, 64], init_state=True, a_mean=-2.0)
    inp["has_init"] = np.array([1, 0, 0, 1], np.int32)
    r1 = _both(g, inp)
    _same(*r1)
    print("static-workspace prefill: call 2, lengths [100]", flush=True)
    inp2 = gi.prefill_inputs(seed=902, geom=g, lengths=[100], init_state=True, a_mean=-2.0)
    r2 = _both(g, inp2)
    _same(*r2)
    assert not torch.isnan(r2[1][0].float()).any()


def test_static_workspace_small_geometry_fp32():
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=1, n_v_heads=3, d_k=32, d_v=32, n_slots=3,
                            dtype_in=gi.F32, dtype_out=gi.F32)
    for seed, lengths in ((903, [257, 70]), (904, [5])):
        print(f"static-workspace prefill: fp32 d=32, lengths {lengths}", flush=True)
        inp = gi.prefill_inputs(seed=seed, geom=g, lengths=lengths, init_state=True)
        _same(*_both(g, inp))
