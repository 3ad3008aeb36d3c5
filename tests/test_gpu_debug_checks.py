"""The debug build of the library (libgdn_debug.so, the C ABI built with
GDN_DEBUG_CHECKS): before a call's kernels it checks on the device that the
call's slot ids are distinct and writes GDN_DEV_DUP_SLOT otherwise; with
distinct ids its results equal the release library's bit for bit."""
import contextlib
import dataclasses
import os

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


@contextlib.contextmanager
def _debug_library(gdn):
    """The binding's calls go to libgdn_debug.so inside the block."""
    saved = gdn._lib, gdn.LIB_PATH
    gdn._lib = None
    gdn.LIB_PATH = os.path.join(os.path.dirname(saved[1]), "libgdn_debug.so")
    try:
        assert b"debug checks" in gdn.lib().gdn_version()
        yield
    finally:
        gdn._lib, gdn.LIB_PATH = saved


def _decode_setup(gdn, slots):
    inp = gi.workload(2)
    g = inp["geom"]
    dt = H.in_dtype(g)
    B = len(slots)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    x, a, b = (H.dev(inp[n][:B, 0], dt) for n in ("x", "a", "b"))
    o = torch.empty(B, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    return g, pool, (x, a, b, H.dev(inp["conv_w"]), H.dev(np.asarray(slots, np.int32))), o


def test_decode_duplicate_slots_reported_distinct_ones_unchanged():
    gdn = _gdn()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g, pool, args, o = _decode_setup(gdn, [0, 1, 2, 3])
    geom = H.to_geom(g)
    gdn.decode_step(geom, pool, *args, o, dev_err=err)  # release library
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, pool.state, pool.conv_state, pool.conv_pos)]
    g, pool, args, o = _decode_setup(gdn, [0, 1, 2, 3])
    with _debug_library(gdn):
        gdn.decode_step(geom, pool, *args, o, dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        for i, (a, b) in enumerate(zip((o, pool.state, pool.conv_state, pool.conv_pos), ref)):
            assert torch.equal(a, b), f"result {i} of the debug library differs"
        g, pool, args, o = _decode_setup(gdn, [0, 1, 1, 3])
        gdn.decode_step(geom, pool, *args, o, dev_err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == gdn.DEV_DUP_SLOT
    # the release library does not check
    err.zero_()
    g, pool, args, o = _decode_setup(gdn, [0, 1, 1, 3])
    gdn.decode_step(geom, pool, *args, o, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


def test_verify_slots_checks_only_the_snapshots_a_row_uses():
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=8)
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    inp = gi.workload(5)
    k = 2
    pool = gdn.SlotPool.zeros(geom)
    x, a, b = (H.dev(inp[n][:2, :k], dt) for n in ("x", "a", "b"))
    cw = H.dev(inp["conv_w"])
    slot = H.dev(np.array([0, 1], np.int32))
    o = torch.empty(2, k, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cases = [([[2, 3], [4, 5]], None, 0),   # distinct
             ([[2, 3], [4, 0]], None, 7),   # row 1's second snapshot is row 0's slot
             ([[2, 3], [4, 0]], [2, 1], 0),  # ... but row 1 makes one draft: that entry is unused
             ([[2, 3], [3, 5]], [2, 1], 7)]  # two rows' snapshots in one slot
    with _debug_library(gdn):
        for ss, k_row, want in cases:
            err.zero_()
            kr = None if k_row is None else H.dev(np.asarray(k_row, np.int32))
            gdn.verify_k_slots(geom, pool, x, a, b, cw, slot, H.dev(np.asarray(ss, np.int32)), o, dev_err=err,
                               k_row=kr)
            torch.cuda.synchronize()
            assert int(err.item()) == want, (ss, k_row)


def test_prefill_duplicate_slots_reported():
    gdn = _gdn()
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=4)
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    inp = gi.prefill_inputs(seed=970, geom=g, lengths=[100, 70])
    N = inp["x"].shape[0]
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    o = torch.empty(N, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    ws = gdn.alloc_prefill_workspace(geom, N, 2)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with _debug_library(gdn):
        for slots, want in (([1, 2], 0), ([2, 2], 7)):
            err.zero_()
            gdn.prefill_chunked(geom, pool, H.dev(inp["x"], dt), H.dev(inp["a"], dt), H.dev(inp["b"], dt),
                                H.dev(inp["conv_w"]), H.dev(inp["cu_seqlens"]), H.dev(np.asarray(slots, np.int32)),
                                H.dev(inp["has_init"]), o, ws, dev_err=err)
            torch.cuda.synchronize()
            assert int(err.item()) == want, slots
