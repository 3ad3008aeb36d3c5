"""The fp64 oracle's prefill on full-size problems, one k-head group per
worker process.

After the front end, v-heads do not interact, and the front end itself works
channel by channel (conv, SiLU) and head by head (the norms of q and k).  So
the layer restricted to one k-head kh and some of its v-heads is the same
layer on a smaller geometry (1 k-head, those v-heads) whose channels are q of
kh, k of kh and v of those heads, in that order, with the matching columns of
the gate inputs and slices of the state and conv history.  Each worker runs
the unchanged oracle on such a sub-problem; the parent puts the pieces back.

Test infrastructure, like the oracle itself: only the tests and the
benchmark's CPU-baseline leg use it.  The workers import numpy and the
oracle, nothing that touches a GPU; they are started with the "spawn" method
(a fresh interpreter, no copy of a process that holds a GPU context), one
BLAS thread each, at most 16 of them.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import types
from concurrent.futures import ProcessPoolExecutor

import numpy as np

MAX_WORKERS = 16
_FIELDS = ("n_k_heads", "n_v_heads", "d_k", "d_v", "conv_width", "conv_ring", "max_draft", "n_slots",
           "l2norm_qk", "q_scale", "l2_eps")


def _geometry(fields: dict):
    """A plain stand-in for the geometry dataclass with the attributes the oracle reads."""
    g = types.SimpleNamespace(**fields)
    g.conv_channels = 2 * g.n_k_heads * g.d_k + g.n_v_heads * g.d_v
    g.group = g.n_v_heads // g.n_k_heads
    return g


def ping(_):
    """A no-op job: mapping it over the pool starts the workers."""
    return os.getpid()


def init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass


def _run(job):
    from oracle import gdn_oracle as orc
    fields, x, a, b, conv_w, cu, S0, h0, has_init = job
    return orc.prefill(_geometry(fields), x, a, b, conv_w, cu, S0, h0, has_init)


def make_pool(workers=None) -> ProcessPoolExecutor:
    """A pool of spawned oracle workers: at most 16, at most the host's CPUs."""
    n = max(1, min(MAX_WORKERS, workers or MAX_WORKERS, os.cpu_count() or 1))
    return ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=init_worker)


def channels(g, kh: int, heads) -> np.ndarray:
    """Channel indices of the sub-problem of k-head kh with v-heads ``heads``."""
    D, Hk = g.d_k, g.n_k_heads
    parts = [np.arange(kh * D, (kh + 1) * D), np.arange(Hk * D + kh * D, Hk * D + (kh + 1) * D)]
    parts += [np.arange(2 * Hk * D + h * g.d_v, 2 * Hk * D + (h + 1) * g.d_v) for h in heads]
    return np.concatenate(parts)


def prefill_by_groups(g, inp, heads_of_group=None, workers=None, executor=None):
    """orc.prefill on ``inp`` (a prefill_inputs dict) for the v-heads chosen per
    k-head group (all of them by default), computed per group in parallel.

    heads_of_group(kh) -> list of v-heads of group kh.  Returns (o, finals, heads)
    with o (N, len(heads), d_v), finals[s] = (S_T (len(heads), d_v, d_k),
    hist_T (W-1, C) with the channels no chosen head reads left as NaN) and
    heads the v-heads in the order of o's second axis.  ``executor``: a
    running process pool to use (one is made and shut down otherwise).
    """
    G = g.n_v_heads // g.n_k_heads
    pick = heads_of_group or (lambda kh: list(range(kh * G, (kh + 1) * G)))
    S = len(inp["cu_seqlens"]) - 1
    S0 = np.stack([inp["state"][s] for s in inp["slots"]])
    h0 = np.stack([inp["hist"][s] for s in inp["slots"]])
    jobs, layout = [], []
    for kh in range(g.n_k_heads):
        hs = list(pick(kh))
        assert all(kh * G <= h < (kh + 1) * G for h in hs), "heads must belong to the group"
        ch = channels(g, kh, hs)
        fields = {f: getattr(g, f) for f in _FIELDS}
        fields.update(n_k_heads=1, n_v_heads=len(hs))
        jobs.append((fields, np.ascontiguousarray(inp["x"][:, ch]), np.ascontiguousarray(inp["a"][:, hs]),
                     np.ascontiguousarray(inp["b"][:, hs]), np.ascontiguousarray(inp["conv_w"][ch]),
                     inp["cu_seqlens"], np.ascontiguousarray(S0[:, hs]), np.ascontiguousarray(h0[:, :, ch]),
                     inp["has_init"]))
        layout.append((hs, ch))
    if executor is not None:
        results = list(executor.map(_run, jobs))
    else:
        with make_pool(min(len(jobs), workers or MAX_WORKERS)) as ex:
            results = list(ex.map(_run, jobs))
    heads = [h for hs, _ in layout for h in hs]
    N = inp["x"].shape[0]
    o = np.empty((N, len(heads), g.d_v))
    finals = [(np.empty((len(heads), g.d_v, g.d_k)), np.full((max(g.conv_width - 1, 0), g.conv_channels), np.nan))
              for _ in range(S)]
    col = 0
    for (hs, ch), (o_g, fin_g) in zip(layout, results):
        o[:, col:col + len(hs)] = o_g
        for s in range(S):
            finals[s][0][col:col + len(hs)] = fin_g[s][0]
            finals[s][1][:, ch] = fin_g[s][1]
        col += len(hs)
    return o, finals, heads
