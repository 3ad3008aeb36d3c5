"""Test harness: moves seeded inputs to the device, lays out the slot pool the
way include/gdn.h documents it, and compares GPU results with the oracle.

It holds no layer arithmetic: the conv ring helpers only place and read back
rows (ring row of token p is p mod R; conv_pos counts tokens x 65536).
"""
from __future__ import annotations

import numpy as np
import torch

import gdn_inputs as gi

TOL_F32 = 1e-4   # fp32 inputs, fp32 state
TOL_BF16 = 2e-2  # bf16 inputs, fp32 state


def tol_for(geom: gi.Geometry) -> float:
    return TOL_BF16 if geom.dtype_in == gi.BF16 else TOL_F32


def relerr(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor (normwise, per tensor)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    if den == 0.0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


def to_geom(g: gi.Geometry):
    import gated_deltanet_delta_amd as gdn
    return gdn.Geometry(n_k_heads=g.n_k_heads, n_v_heads=g.n_v_heads, d_k=g.d_k, d_v=g.d_v,
                        conv_width=g.conv_width, conv_ring=g.conv_ring, max_draft=g.max_draft,
                        n_slots=g.n_slots, dtype=torch.bfloat16 if g.dtype_in == gi.BF16 else torch.float32,
                        l2norm_qk=g.l2norm_qk, q_scale=g.q_scale, l2_eps=g.l2_eps)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def in_dtype(g: gi.Geometry):
    return torch.bfloat16 if g.dtype_in == gi.BF16 else torch.float32


def make_pool(g: gi.Geometry, state, hist, pos):
    """SlotPool holding `state` (n_slots,H,dv,dk), history `hist` (n_slots,W-1,C)
    at ring positions `pos` (n_slots,) tokens."""
    import gated_deltanet_delta_amd as gdn
    geom = to_geom(g)
    pool = gdn.SlotPool.zeros(geom)
    pool.state.copy_(torch.from_numpy(np.ascontiguousarray(state, np.float32)))
    W, R = g.conv_width, g.conv_ring
    if W > 0:
        ring = np.zeros((g.n_slots, R, g.conv_channels), np.float32)
        for s in range(g.n_slots):
            for i in range(W - 1):  # hist row i is token pos-(W-1)+i
                ring[s, (int(pos[s]) - (W - 1) + i) % R] = hist[s, i]
        pool.conv_state.copy_(torch.from_numpy(ring))
        pool.conv_pos[:, 0].copy_(torch.from_numpy((np.asarray(pos, np.int64) * gi_pos_one()).astype(np.int32)))
    return pool


def gi_pos_one() -> int:
    import gated_deltanet_delta_amd as gdn
    return gdn.POS_ONE


def positions(pool) -> np.ndarray:
    """Token positions of every slot (conv_pos / 65536, as unsigned)."""
    p = pool.conv_pos[:, 0].cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    return p >> 16


def read_hist(g: gi.Geometry, pool) -> np.ndarray:
    """Conv history (n_slots, W-1, C), oldest first, read from the ring."""
    W, R = g.conv_width, g.conv_ring
    ring = pool.conv_state.cpu().numpy()
    pos = positions(pool)
    out = np.zeros((g.n_slots, max(W - 1, 0), g.conv_channels), np.float32)
    for s in range(g.n_slots):
        for i in range(W - 1):
            out[s, i] = ring[s, (int(pos[s]) - (W - 1) + i) % R]
    return out


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
