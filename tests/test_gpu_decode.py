"""Decode step and conv-ring step on the GPU against the fp64 oracle."""
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


def _run_decode(g, inp, steps=1):
    """Run `steps` decode tokens (the same seeded row block re-drawn per step)
    on the GPU and in the oracle; return both results."""
    gdn = _gdn()
    geom = H.to_geom(g)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    dt = H.in_dtype(g)
    slots = H.dev(inp["slots"])
    conv_w = H.dev(inp["conv_w"]) if g.conv_width else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    st, hi = np.array(inp["state"], np.float64), np.array(inp["hist"], np.float64)
    outs_gpu, outs_ref = [], []
    B = len(inp["slots"])
    for t in range(steps):
        x, a, b = inp["x"][:, t], inp["a"][:, t], inp["b"][:, t]
        o = torch.empty(B, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
        gdn.decode_step(geom, pool, H.dev(x, dt), H.dev(a, dt), H.dev(b, dt), conv_w, slots, o, dev_err=err)
        outs_gpu.append(H.f64(o))
        o_ref, st, hi = orc.decode_step(g, st, hi, x, a, b, inp["conv_w"], inp["slots"])
        outs_ref.append(o_ref)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return pool, np.stack(outs_gpu), np.stack(outs_ref), st, hi


def test_decode_workload2_full():
    """4 slots x 1 token, 16/48 heads, d = 128, bf16 inputs: o and states within 2e-2,
    untouched slots bitwise unchanged, ring history exact, position +1."""
    inp = gi.workload(2)
    g = inp["geom"]
    pool, o_gpu, o_ref, st_ref, hi_ref = _run_decode(g, inp)
    assert H.relerr(o_gpu, o_ref) <= H.TOL_BF16
    state = pool.state.cpu().numpy()
    for s in range(g.n_slots):
        if s in inp["slots"]:
            assert H.relerr(state[s], st_ref[s]) <= H.TOL_BF16, f"slot {s}"
        else:
            assert np.array_equal(state[s], inp["state"][s]), f"untouched slot {s} changed"
    hist = H.read_hist(g, pool)
    assert np.array_equal(hist, hi_ref.astype(np.float32))
    pos = H.positions(pool)
    for s in range(g.n_slots):
        assert pos[s] == inp["pos"][s] + (1 if s in inp["slots"] else 0)
    assert np.all((pool.conv_pos[:, 0].cpu().numpy() & 0xFFFF) == 0)
    assert not pool.conv_pos[:, 1:].any()  # the rest of each slot's line is never written


def test_decode_batch_64():
    """64 slots in one call (the batch sweep's middle size) out of a pool of 66:
    every row's output and state within 2e-2, the two untouched slots bitwise
    unchanged, every position +1."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_slots=66)
    inp = gi.decode_inputs(seed=140, geom=g, batch=64)
    pool, o_gpu, o_ref, st_ref, hi_ref = _run_decode(g, inp)
    assert H.relerr(o_gpu, o_ref) <= H.TOL_BF16
    state = pool.state.cpu().numpy()
    for s in range(g.n_slots):
        if s in inp["slots"]:
            assert H.relerr(state[s], st_ref[s]) <= H.TOL_BF16, f"slot {s}"
        else:
            assert np.array_equal(state[s], inp["state"][s]), f"untouched slot {s} changed"
    assert np.array_equal(H.read_hist(g, pool), hi_ref.astype(np.float32))
    pos = H.positions(pool)
    assert all(pos[s] == inp["pos"][s] + (1 if s in inp["slots"] else 0) for s in range(g.n_slots))


def test_decode_tight_error_bound():
    """The achieved error is far inside the gate (fp32 state, fp32 math)."""
    inp = gi.workload(2, seed=7)
    pool, o_gpu, o_ref, st_ref, _ = _run_decode(inp["geom"], inp)
    assert H.relerr(o_gpu, o_ref) <= 8e-3  # bf16 rounding of o dominates
    s = inp["slots"][0]
    assert H.relerr(pool.state.cpu().numpy()[s], st_ref[s]) <= 1e-5


def test_decode_many_steps_bf16():
    inp = gi.decode_inputs(seed=11, n_tokens=12)
    g = inp["geom"]
    pool, o_gpu, o_ref, st_ref, hi_ref = _run_decode(g, inp, steps=12)
    assert H.relerr(o_gpu, o_ref) <= H.TOL_BF16
    state = pool.state.cpu().numpy()
    for s in inp["slots"]:
        assert H.relerr(state[s], st_ref[s]) <= H.TOL_BF16
    assert np.array_equal(H.read_hist(g, pool), hi_ref.astype(np.float32))


def test_workload1_through_decode_fp32():
    """Tiny fp32 recurrence (d = 16, T = 64, no conv) through 64 decode steps: 1e-4."""
    inp = gi.workload(1)
    g = inp["geom"]
    gdn = _gdn()
    geom = H.to_geom(g)
    pool = gdn.SlotPool.zeros(geom)
    slots = H.dev(np.array([0], np.int32))
    T = inp["x"].shape[0]
    o_all = []
    for t in range(T):
        o = torch.empty(1, 1, 16, dtype=torch.float32, device="cuda")
        gdn.decode_step(geom, pool, H.dev(inp["x"][t:t + 1]), H.dev(inp["a"][t:t + 1]),
                        H.dev(inp["b"][t:t + 1]), None, slots, o)
        o_all.append(H.f64(o)[0])
    o_ref, S_ref, _ = orc.layer_sequence(g, inp["x"], inp["a"], inp["b"], inp["conv_w"],
                                         np.zeros((1, 16, 16)), np.zeros((0, g.conv_channels)))
    assert H.relerr(np.stack(o_all), o_ref) <= H.TOL_F32
    assert H.relerr(pool.state.cpu().numpy()[0], S_ref) <= H.TOL_F32


@pytest.mark.parametrize("d,hk,G", [(16, 2, 3), (32, 3, 1), (64, 2, 4), (128, 1, 2)])
@pytest.mark.parametrize("dtype", [gi.BF16, gi.F32])
def test_decode_geometries(d, hk, G, dtype):
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=hk, n_v_heads=hk * G, d_k=d, d_v=d, n_slots=5,
                            dtype_in=dtype, dtype_out=dtype, q_scale=0.5)
    inp = gi.decode_inputs(seed=100 + d + G, geom=g, batch=3, n_tokens=3)
    pool, o_gpu, o_ref, st_ref, hi_ref = _run_decode(g, inp, steps=3)
    tol = H.tol_for(g)
    assert H.relerr(o_gpu, o_ref) <= tol
    state = pool.state.cpu().numpy()
    for s in inp["slots"]:
        assert H.relerr(state[s], st_ref[s]) <= tol
    assert np.array_equal(H.read_hist(g, pool), hi_ref.astype(np.float32))


def test_decode_deterministic_and_batch_invariant():
    """Same inputs twice: bitwise equal; a slot's result does not depend on its
    batch position or on the other rows of the batch."""
    gdn = _gdn()
    inp = gi.workload(2, seed=21)
    g = inp["geom"]
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    x, a, b = (H.dev(inp[k][:, 0], dt) for k in ("x", "a", "b"))
    cw = H.dev(inp["conv_w"])

    def run(order):
        pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
        idx = torch.tensor(order, device="cuda")
        o = torch.empty(len(order), g.n_v_heads, g.d_v, dtype=dt, device="cuda")
        gdn.decode_step(geom, pool, x[idx].contiguous(), a[idx].contiguous(), b[idx].contiguous(), cw,
                        H.dev(inp["slots"][order]), o)
        return pool.state.cpu(), o.cpu()[np.argsort(order)] if len(order) == 4 else o.cpu()

    s1, o1 = run([0, 1, 2, 3])
    s2, o2 = run([0, 1, 2, 3])
    assert torch.equal(s1, s2) and torch.equal(o1, o2)
    s3, o3 = run([3, 1, 0, 2])
    assert torch.equal(s1, s3) and torch.equal(o1, o3)
    s4, o4 = run([2])
    assert torch.equal(o4[0], o1[2])
    slot2 = int(inp["slots"][2])
    assert torch.equal(s4[slot2], s1[slot2])


def test_decode_bad_slot_is_reported_and_skipped():
    gdn = _gdn()
    inp = gi.workload(2, seed=5)
    g = inp["geom"]
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    before = pool.state.clone()
    pos_before = pool.conv_pos.clone()
    slots = inp["slots"].copy()
    slots[1] = g.n_slots + 3
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.zeros(4, g.n_v_heads, g.d_v, dtype=dt, device="cuda")
    gdn.decode_step(geom, pool, H.dev(inp["x"][:, 0], dt), H.dev(inp["a"][:, 0], dt),
                    H.dev(inp["b"][:, 0], dt), H.dev(inp["conv_w"]), H.dev(slots), o, dev_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gdn.DEV_BAD_SLOT
    # the valid rows were processed, the bad one left everything alone
    for i, s in enumerate(slots):
        if i == 1:
            continue
        assert not torch.equal(pool.state[s], before[s])
    assert torch.all(o[1].float() == 0)
    changed = (pool.conv_pos != pos_before).sum().item()
    assert changed == 3


def test_conv_state_step_matches_oracle():
    gdn = _gdn()
    inp = gi.decode_inputs(seed=31, n_tokens=5)
    g = inp["geom"]
    geom = H.to_geom(g)
    dt = H.in_dtype(g)
    pool = H.make_pool(g, inp["state"], inp["hist"], inp["pos"])
    hist = np.array(inp["hist"], np.float64)
    slots = H.dev(inp["slots"])
    for t in range(5):
        y = torch.empty(4, g.conv_channels, dtype=dt, device="cuda")
        gdn.conv_state_step(geom, pool, H.dev(inp["x"][:, t], dt), H.dev(inp["conv_w"]), slots, y)
        for i, s in enumerate(inp["slots"]):
            window = np.concatenate([hist[s], inp["x"][i, t][None].astype(np.float64)])
            ref = orc.conv_silu(window, inp["conv_w"])
            assert H.relerr(H.f64(y[i]), ref) <= 8e-3
            hist[s] = window[1:]
    torch.cuda.synchronize()
    assert np.array_equal(H.read_hist(g, pool), hist.astype(np.float32))
    assert np.array_equal(pool.state.cpu().numpy(), inp["state"])  # state untouched


def test_decode_extreme_gates():
    """Decode with gate inputs at -40 / 40 (exact in bf16): alpha = 1 or e^-40,
    beta = e^-40 or 1, over several tokens."""
    g = dataclasses.replace(gi.GEOM_QWEN, n_k_heads=2, n_v_heads=6, n_slots=4)
    inp = gi.decode_inputs(seed=150, geom=g, batch=3, n_tokens=4)
    rng = np.random.Generator(np.random.PCG64(151))
    vals = np.array([-40.0, 40.0], np.float32)
    inp["a"] = vals[rng.integers(0, 2, size=inp["a"].shape)]
    inp["b"] = vals[rng.integers(0, 2, size=inp["b"].shape)]
    pool, o_gpu, o_ref, st_ref, _ = _run_decode(g, inp, steps=4)
    assert np.isfinite(o_gpu).all()
    assert H.relerr(o_gpu, o_ref) <= H.TOL_BF16
    for s in inp["slots"]:
        assert H.relerr(pool.state[s].cpu().numpy(), st_ref[s]) <= H.TOL_BF16
