"""Seeded synthetic inputs for the Gated DeltaNet layer.

This module only draws random numbers and lays them out.  It holds none of
the layer's arithmetic: no convolution, no normalisation, no gate law, no
state update.  Both the CPU oracle (``oracle/``) and the HIP path (through
its Python binding) receive the very same arrays from here.

Shapes and value distributions follow the five workloads of the layer:

  1. tiny fp32 recurrence: 1 k-head / 1 v-head, d = 16, T = 64, no conv,
     q and k drawn from N(0,1) then scaled to unit length per token;
  2. decode: 4 active slots of a pool of 8, one token each, 16 k-heads,
     48 v-heads, d = 128, C = 10240 conv channels, bf16 inputs;
  3. chunked prefill of one sequence of T = 8192, zero initial state;
  4. variable-length prefill of 4 sequences, lengths uniform in
     [1024, 32768], nonzero initial state and conv history, long-memory
     gates (the gate pre-activation a ~ N(-2, 1));
  5. speculative verify of k = 4 drafts on 4 slots, then rollback to a
     seeded accepted length in {0..4}.

The head geometry (16 k-heads, 48 v-heads, state 128, conv width 4,
10240 conv channels = 2*128*16 + 128*48) is the GDN geometry printed in
"Chapter 6: engine startup and memory plan" (Strata book), section 6.2.

Random draws use numpy's PCG64 seeded with the workload index unless a
seed is given; the draw order inside each recipe is fixed and listed in
the recipe.  bf16 inputs are produced by rounding fp32 draws to nearest
even (torch's fp32 -> bf16 cast) and are handed to both sides as the
rounded values, so the oracle reads exactly what the GPU reads.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

@dataclasses.dataclass(frozen=True)
class Geometry:
    """Sizes of one GDN layer instance (all of them are kernel contracts)."""

    n_k_heads: int = 16
    n_v_heads: int = 48
    d_k: int = 128
    d_v: int = 128
    conv_width: int = 4
    conv_ring: int = 8
    max_draft: int = 4
    n_slots: int = 8
    dtype_in: str = BF16
    dtype_out: str = BF16
    l2norm_qk: bool = True
    q_scale: float = 1.0
    l2_eps: float = 1e-6

    @property
    def conv_channels(self) -> int:
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v

    @property
    def group(self) -> int:
        return self.n_v_heads // self.n_k_heads


GEOM_QWEN = Geometry()
GEOM_TINY = Geometry(n_k_heads=1, n_v_heads=1, d_k=16, d_v=16, conv_width=0,
                     conv_ring=8, max_draft=4, n_slots=1, dtype_in=F32,
                     dtype_out=F32, l2norm_qk=False)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 (nearest even) and return it as fp32."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _cast_in(a: np.ndarray, geom: Geometry) -> np.ndarray:
    a = a.astype(np.float32)
    return round_bf16(a) if geom.dtype_in == BF16 else a


def _normal(rng, shape, mean=0.0, std=1.0):
    return rng.normal(mean, std, size=shape).astype(np.float32)


def _unit_rows(v: np.ndarray) -> np.ndarray:
    """Scale each row (last axis) of a draw to unit length, computed in fp64.

    This shapes the random draw for workload 1 (its q and k are defined as
    unit vectors); it is not the layer's own normalisation step.
    """
    v64 = v.astype(np.float64)
    n = np.sqrt((v64 * v64).sum(axis=-1, keepdims=True))
    return (v64 / n).astype(np.float32)


def tiny_inputs(seed: int = 0, T: int = 64, d: int = 16, n_heads: int = 1):
    """Workload 1: plain recurrence, no conv, fp32.

    Draw order: q (T,H,d), k (T,H,d), v (T,H,d), a (T,H), b (T,H).
    x packs q | k | v along channels so it has the layout the layer takes
    when the conv is switched off.
    """
    geom = dataclasses.replace(GEOM_TINY, n_k_heads=n_heads, n_v_heads=n_heads,
                               d_k=d, d_v=d)
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _unit_rows(_normal(rng, (T, n_heads, d)))
    k = _unit_rows(_normal(rng, (T, n_heads, d)))
    v = _normal(rng, (T, n_heads, d))
    a = _normal(rng, (T, n_heads))
    b = _normal(rng, (T, n_heads))
    x = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    return dict(geom=geom, x=x.astype(np.float32), a=a, b=b,
                conv_w=np.zeros((geom.conv_channels, 0), np.float32),
                state0=np.zeros((1, n_heads, d, d), np.float32),
                cu_seqlens=np.array([0, T], np.int32), slots=np.array([0], np.int32),
                has_init=np.array([0], np.int32))


def _pool(rng, geom: Geometry, state_std: float, hist_std: float):
    """A slot pool: states (n_slots,H_v,d_v,d_k) and conv histories (n_slots,W-1,C)."""
    st = _normal(rng, (geom.n_slots, geom.n_v_heads, geom.d_v, geom.d_k), std=state_std)
    hist = _normal(rng, (geom.n_slots, max(geom.conv_width - 1, 0), geom.conv_channels),
                   std=hist_std)
    return st, hist


def decode_inputs(seed: int = 1, geom: Geometry = GEOM_QWEN, batch: int = 4,
                  n_tokens: int = 1):
    """Workload 2 (n_tokens = 1) and the draft block of workload 5 (n_tokens = k).

    Draw order: slot ids (distinct, from the pool), conv weights (C,W) ~ N(0,0.5),
    pool states ~ N(0,0.02), pool conv histories ~ N(0,0.1),
    x (B,n,C) ~ N(0,1), a (B,n,H_v) ~ N(0,1), b (B,n,H_v) ~ N(0,1),
    accepted lengths (B,) uniform in {0..n}.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    slots = rng.choice(geom.n_slots, size=batch, replace=False).astype(np.int32)
    conv_w = _normal(rng, (geom.conv_channels, geom.conv_width), std=0.5)
    state, hist = _pool(rng, geom, 0.02, 0.1)
    x = _cast_in(_normal(rng, (batch, n_tokens, geom.conv_channels)), geom)
    a = _cast_in(_normal(rng, (batch, n_tokens, geom.n_v_heads)), geom)
    b = _cast_in(_normal(rng, (batch, n_tokens, geom.n_v_heads)), geom)
    accepted = rng.integers(0, n_tokens, size=batch, endpoint=True).astype(np.int32)
    pos = rng.integers(0, 1 << 12, size=geom.n_slots).astype(np.int64)
    return dict(geom=geom, slots=slots, conv_w=conv_w, state=state, hist=hist,
                x=x, a=a, b=b, accepted=accepted, pos=pos)


def verify_inputs(seed: int = 4, geom: Geometry = GEOM_QWEN, batch: int = 4, k: int = 4):
    """Workload 5: k drafts per slot, same recipe as workload 2."""
    return decode_inputs(seed=seed, geom=geom, batch=batch, n_tokens=k)


def prefill_inputs(seed: int = 2, geom: Geometry = GEOM_QWEN,
                   lengths: Optional[list] = None, a_mean: float = 0.0,
                   init_state: bool = False, n_seqs: int = 1,
                   len_range: tuple = (1024, 32768)):
    """Workloads 3 and 4 (and smaller cases of the same recipe).

    Draw order: sequence lengths (if not given; uniform inclusive in len_range),
    slot ids (distinct), conv weights (C,W) ~ N(0,0.5), pool states ~ N(0,0.02)
    and conv histories ~ N(0,0.1) (drawn always, used only when init_state),
    x (N,C) ~ N(0,1), a (N,H_v) ~ N(a_mean,1), b (N,H_v) ~ N(0,1).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if lengths is None:
        lengths = rng.integers(len_range[0], len_range[1], size=n_seqs, endpoint=True).tolist()
    lengths = [int(x) for x in lengths]
    S = len(lengths)
    cu = np.zeros(S + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    N = int(cu[-1])
    slots = rng.choice(geom.n_slots, size=S, replace=False).astype(np.int32)
    conv_w = _normal(rng, (geom.conv_channels, geom.conv_width), std=0.5)
    state, hist = _pool(rng, geom, 0.02, 0.1)
    x = _cast_in(_normal(rng, (N, geom.conv_channels)), geom)
    a = _cast_in(_normal(rng, (N, geom.n_v_heads), mean=a_mean), geom)
    b = _cast_in(_normal(rng, (N, geom.n_v_heads)), geom)
    has_init = np.full(S, 1 if init_state else 0, np.int32)
    pos = rng.integers(0, 1 << 12, size=geom.n_slots).astype(np.int64)
    return dict(geom=geom, lengths=lengths, cu_seqlens=cu, slots=slots, conv_w=conv_w,
                state=state, hist=hist, x=x, a=a, b=b, has_init=has_init, pos=pos)


def workload(index: int, seed: Optional[int] = None, **kw):
    """The five workloads by 1-based index, seed defaulting to the index."""
    seed = index if seed is None else seed
    if index == 1:
        return tiny_inputs(seed=seed, **kw)
    if index == 2:
        return decode_inputs(seed=seed, **kw)
    if index == 3:
        kw.setdefault("lengths", [8192])
        return prefill_inputs(seed=seed, **kw)
    if index == 4:
        kw.setdefault("n_seqs", 4)
        kw.setdefault("a_mean", -2.0)
        kw.setdefault("init_state", True)
        return prefill_inputs(seed=seed, **kw)
    if index == 5:
        return verify_inputs(seed=seed, **kw)
    raise ValueError(f"no workload {index}")
