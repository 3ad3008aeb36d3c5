"""Gated DeltaNet layer for AMD MI355X (gfx950): Python binding of libgdn.so.

This module only marshals arguments: it checks tensor shapes, dtypes and
devices on the host (so that no kernel is launched on buffers smaller than
its grid assumes), then passes raw device pointers and the current HIP stream
to the C ABI declared in include/gdn.h.  Every step of the layer runs in the
library's HIP kernels; there is no fallback.  If libgdn.so has not been built
the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
GDN_FLAG_L2NORM_QK = 1
POS_ONE = 65536
POS_STRIDE = 32  # int32 words per slot in conv_pos: slot s's position is conv_pos[s, 0]
CHUNK = 64

ABI_VERSION = 7  # GDN_ABI_VERSION of include/gdn.h that these signatures follow
DEV_OK = 0
DEV_BAD_SLOT = 1
DEV_BAD_ACCEPTED = 2
DEV_BAD_SEQLENS = 3
DEV_WAIT_TIMEOUT = 4
DEV_BAD_K = 5
DEV_INCOMPLETE = 6
DEV_DUP_SLOT = 7  # libgdn_debug.so only


class GdnGeometry(ctypes.Structure):
    _fields_ = [
        ("n_k_heads", ctypes.c_int32),
        ("n_v_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("conv_channels", ctypes.c_int32),
        ("conv_ring", ctypes.c_int32),
        ("max_draft", ctypes.c_int32),
        ("n_slots", ctypes.c_int32),
        ("dtype_in", ctypes.c_int32),
        ("dtype_out", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("q_scale", ctypes.c_float),
        ("l2_eps", ctypes.c_float),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, name: str, message: str):
        super().__init__(f"{name}: {message}")
        self.status = status
        self.name = name
        self.message = message


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "gdn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdn_last_error": (ctypes.c_char_p, []),
    "gdn_version": (ctypes.c_char_p, []),
    "gdn_abi_version": (ctypes.c_int32, []),
    "gdn_check_geometry": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), ctypes.c_char_p, ctypes.c_size_t]),
    "gdn_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(GdnGeometry), _I, _I]),
    "gdn_conv_state_step": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _I, _P, _P, _P]),
    "gdn_decode_step": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _P, _P, _P, _I,
                                       _P, _P, _P]),
    "gdn_prefill_chunked": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _I, _I, _I, _P, ctypes.c_size_t, _P, _P, _P]),
    "gdn_prefill_chunked_ckpt": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _P, _P, _P,
                                                _P, _P, _I, _I, _I, _P, ctypes.c_size_t, _P, _I, _P,
                                                ctypes.c_size_t, _P, _P]),
    "gdn_prefill_chunked_static": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _P, _P, _P,
                                                  _P, _P, _I, _I, _I, _P, _P, _P]),
    "gdn_verify_k": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _P, _P, _P, _I, _I,
                                    _P, _P, _P, _P]),
    "gdn_rollback": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _I, _I, _P, _P]),
    "gdn_verify_k_slots": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _P, _P, _P, _P, _I, _I,
                                          _P, _P, _P, _P, _P]),
    "gdn_commit_slots": (ctypes.c_int, [ctypes.POINTER(GdnGeometry), _P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "gdn_prefill_timing_events": (ctypes.c_int, [_P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m gated_deltanet_delta_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if L.gdn_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.gdn_abi_version()}, this binding needs "
                               f"{ABI_VERSION}; rebuild it with __graft_entry__.build()")
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        L = lib()
        raise GdnError(status, L.gdn_status_string(status).decode(), L.gdn_last_error().decode())


# --------------------------------------------------------------------------
# geometry
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Geometry:
    """Python mirror of gdn_geometry (see include/gdn.h for every field)."""

    n_k_heads: int = 16
    n_v_heads: int = 48
    d_k: int = 128
    d_v: int = 128
    conv_width: int = 4
    conv_ring: int = 8
    max_draft: int = 4
    n_slots: int = 8
    dtype: torch.dtype = torch.bfloat16
    l2norm_qk: bool = True
    q_scale: float = 1.0
    l2_eps: float = 1e-6

    @property
    def conv_channels(self) -> int:
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v

    def c_struct(self) -> GdnGeometry:
        code = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}[self.dtype]
        return GdnGeometry(self.n_k_heads, self.n_v_heads, self.d_k, self.d_v, self.conv_width,
                           self.conv_channels, self.conv_ring, self.max_draft, self.n_slots, code, code,
                           GDN_FLAG_L2NORM_QK if self.l2norm_qk else 0, self.q_scale, self.l2_eps)

    def check(self):
        g = self.c_struct()
        _check(lib().gdn_check_geometry(ctypes.byref(g), None, 0))


# --------------------------------------------------------------------------
# host-side marshalling helpers
# --------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, shape, dtype, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: missing")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, required {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, required {tuple(shape)}")


@dataclass
class SlotPool:
    """Caller-owned device buffers of one layer's slot pool."""

    state: torch.Tensor       # fp32 [n_slots][H_v][d_v][d_k]
    conv_state: torch.Tensor  # fp32 [n_slots][R][C]
    conv_pos: torch.Tensor    # int32 [n_slots][POS_STRIDE], position in column 0, units of 1/65536 token

    @staticmethod
    def zeros(geom: Geometry, device="cuda") -> "SlotPool":
        C, R = geom.conv_channels, max(geom.conv_ring, 1)
        return SlotPool(
            torch.zeros(geom.n_slots, geom.n_v_heads, geom.d_v, geom.d_k, dtype=torch.float32, device=device),
            torch.zeros(geom.n_slots, R, C, dtype=torch.float32, device=device),
            torch.zeros(geom.n_slots, POS_STRIDE, dtype=torch.int32, device=device))


def _check_pool(geom: Geometry, pool: SlotPool):
    _need(pool.state, "state", (geom.n_slots, geom.n_v_heads, geom.d_v, geom.d_k), torch.float32)
    if geom.conv_width > 0:
        _need(pool.conv_state, "conv_state", (geom.n_slots, geom.conv_ring, geom.conv_channels), torch.float32)
        _need(pool.conv_pos, "conv_pos", (geom.n_slots, POS_STRIDE), torch.int32)


# --------------------------------------------------------------------------
# the five entry points
# --------------------------------------------------------------------------

def conv_state_step(geom: Geometry, pool: SlotPool, x, conv_w, slot, y, dev_err=None, stream=None):
    """gdn_conv_state_step: y = SiLU(causal conv) for all channels; append x to the ring."""
    B = slot.shape[0]
    C = geom.conv_channels
    _check_pool(geom, pool)
    _need(x, "x", (B, C), geom.dtype)
    _need(conv_w, "conv_w", (C, geom.conv_width), torch.float32)
    _need(slot, "slot", (B,), torch.int32)
    _need(y, "y", (B, C), geom.dtype)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    g = geom.c_struct()
    _check(lib().gdn_conv_state_step(ctypes.byref(g), _ptr(pool.conv_state), _ptr(pool.conv_pos), _ptr(x),
                                     _ptr(conv_w), _ptr(slot), B, _ptr(y), _ptr(dev_err), _stream(stream)))


def decode_step(geom: Geometry, pool: SlotPool, x, a, b, conv_w, slot, o, dev_err=None, stream=None):
    """gdn_decode_step: one fused token per batch row; state updated in place."""
    B = slot.shape[0]
    C, Hv, dv = geom.conv_channels, geom.n_v_heads, geom.d_v
    _check_pool(geom, pool)
    _need(x, "x", (B, C), geom.dtype)
    _need(a, "a", (B, Hv), geom.dtype)
    _need(b, "b", (B, Hv), geom.dtype)
    _need(conv_w, "conv_w", (C, geom.conv_width), torch.float32, optional=geom.conv_width == 0)
    _need(slot, "slot", (B,), torch.int32)
    _need(o, "o", (B, Hv, dv), geom.dtype)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    g = geom.c_struct()
    _check(lib().gdn_decode_step(ctypes.byref(g), _ptr(pool.state), _ptr(pool.conv_state), _ptr(pool.conv_pos),
                                 _ptr(x), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(slot), B, _ptr(o),
                                 _ptr(dev_err), _stream(stream)))


def verify_k(geom: Geometry, pool: SlotPool, x, a, b, conv_w, slot, snap, o, dev_err=None, stream=None):
    """gdn_verify_k: k drafts per batch row, snapshot after each; committed state untouched."""
    B, k = x.shape[0], x.shape[1]
    C, Hv, dv, dk = geom.conv_channels, geom.n_v_heads, geom.d_v, geom.d_k
    _check_pool(geom, pool)
    _need(x, "x", (B, k, C), geom.dtype)
    _need(a, "a", (B, k, Hv), geom.dtype)
    _need(b, "b", (B, k, Hv), geom.dtype)
    _need(conv_w, "conv_w", (C, geom.conv_width), torch.float32, optional=geom.conv_width == 0)
    _need(slot, "slot", (B,), torch.int32)
    _need(snap, "snap", (B, k, Hv, dv, dk), torch.float32)
    _need(o, "o", (B, k, Hv, dv), geom.dtype)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    g = geom.c_struct()
    _check(lib().gdn_verify_k(ctypes.byref(g), _ptr(pool.state), _ptr(pool.conv_state), _ptr(pool.conv_pos),
                              _ptr(x), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(slot), B, k, _ptr(snap), _ptr(o),
                              _ptr(dev_err), _stream(stream)))


def rollback(geom: Geometry, pool: SlotPool, snap, slot, accepted, dev_err=None, stream=None):
    """gdn_rollback: commit accepted[i] drafts of batch row i (0 keeps the slot as it was)."""
    B, k = snap.shape[0], snap.shape[1]
    _check_pool(geom, pool)
    _need(snap, "snap", (B, k, geom.n_v_heads, geom.d_v, geom.d_k), torch.float32)
    _need(slot, "slot", (B,), torch.int32)
    _need(accepted, "accepted", (B,), torch.int32)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    g = geom.c_struct()
    _check(lib().gdn_rollback(ctypes.byref(g), _ptr(pool.state), _ptr(pool.conv_pos), _ptr(snap), _ptr(slot),
                              _ptr(accepted), B, k, _ptr(dev_err), _stream(stream)))


def verify_k_slots(geom: Geometry, pool: SlotPool, x, a, b, conv_w, slot, snap_slot, o, dev_err=None,
                   stream=None, k_row=None):
    """gdn_verify_k_slots: as verify_k, but snapshot j of row i becomes pool slot snap_slot[i][j];
    k_row (device int32 [batch], optional) gives each row its own number of drafts."""
    B, k = x.shape[0], x.shape[1]
    C, Hv, dv = geom.conv_channels, geom.n_v_heads, geom.d_v
    _check_pool(geom, pool)
    _need(x, "x", (B, k, C), geom.dtype)
    _need(a, "a", (B, k, Hv), geom.dtype)
    _need(b, "b", (B, k, Hv), geom.dtype)
    _need(conv_w, "conv_w", (C, geom.conv_width), torch.float32, optional=geom.conv_width == 0)
    _need(slot, "slot", (B,), torch.int32)
    _need(snap_slot, "snap_slot", (B, k), torch.int32)
    _need(k_row, "k_row", (B,), torch.int32, optional=True)
    _need(o, "o", (B, k, Hv, dv), geom.dtype)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    g = geom.c_struct()
    _check(lib().gdn_verify_k_slots(ctypes.byref(g), _ptr(pool.state), _ptr(pool.conv_state),
                                    _ptr(pool.conv_pos), _ptr(x), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(slot), B,
                                    k, _ptr(k_row), _ptr(snap_slot), _ptr(o), _ptr(dev_err), _stream(stream)))


def commit_slots(geom: Geometry, slot, snap_slot, accepted, next_slot, dev_err=None, stream=None, k_row=None):
    """gdn_commit_slots: next_slot[i] = snap_slot[i][accepted[i]-1], or slot[i] when accepted[i] == 0."""
    B, k = snap_slot.shape[0], snap_slot.shape[1]
    _need(slot, "slot", (B,), torch.int32)
    _need(k_row, "k_row", (B,), torch.int32, optional=True)
    _need(snap_slot, "snap_slot", (B, k), torch.int32)
    _need(accepted, "accepted", (B,), torch.int32)
    _need(next_slot, "next_slot", (B,), torch.int32)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    g = geom.c_struct()
    _check(lib().gdn_commit_slots(ctypes.byref(g), _ptr(slot), _ptr(k_row), _ptr(snap_slot), _ptr(accepted), B,
                                  k, _ptr(next_slot), _ptr(dev_err), _stream(stream)))


_err_words = {}


def _default_err(device) -> torch.Tensor:
    """The binding's own device error word of a device (prefill calls without
    a dev_err of their own report into it; read it with device_error())."""
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    w = _err_words.get(idx)
    if w is None:
        w = torch.zeros(1, dtype=torch.int32, device=torch.device("cuda", idx))
        _err_words[idx] = w
    return w


def device_error(device="cuda", clear: bool = True) -> int:
    """First device error code the prefill calls without a dev_err of their
    own reported on this device since the last clear (synchronises)."""
    w = _default_err(device)
    v = int(w.item())
    if clear and v:
        w.zero_()
    return v


def prefill_workspace_bytes(geom: Geometry, n_tokens: int, n_seqs: int) -> int:
    g = geom.c_struct()
    return int(lib().gdn_prefill_workspace_bytes(ctypes.byref(g), n_tokens, n_seqs))


def alloc_prefill_workspace(geom: Geometry, n_tokens: int, n_seqs: int, device="cuda") -> torch.Tensor:
    """A caller-owned workspace of the size gdn_prefill_workspace_bytes reports."""
    n = prefill_workspace_bytes(geom, n_tokens, n_seqs)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def prefill_chunked(geom: Geometry, pool: SlotPool, x, a, b, conv_w, cu_seqlens, slot, has_init, o,
                    workspace, dev_err=None, stream=None, ckpt=None, ckpt_every=0):
    """gdn_prefill_chunked: varlen chunked prefill; final states and histories go to the slots.

    With ckpt_every > 0 it calls gdn_prefill_chunked_ckpt instead, which also
    writes the state after every ckpt_every tokens of each sequence into ckpt,
    an fp32 device tensor [n][H_v][d_v][d_k] with n >= n_tokens // ckpt_every
    (see ``checkpoint_count`` for the number a partition produces).
    Without a dev_err of the caller's, device errors go to the binding's own
    word for the device (``device_error``).
    """
    N = x.shape[0]
    S = slot.shape[0]
    C, Hv, dv = geom.conv_channels, geom.n_v_heads, geom.d_v
    _check_pool(geom, pool)
    _need(x, "x", (N, C), geom.dtype)
    _need(a, "a", (N, Hv), geom.dtype)
    _need(b, "b", (N, Hv), geom.dtype)
    _need(conv_w, "conv_w", (C, geom.conv_width), torch.float32, optional=geom.conv_width == 0)
    _need(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32)
    _need(slot, "slot", (S,), torch.int32)
    _need(has_init, "has_init", (S,), torch.int32)
    _need(o, "o", (N, Hv, dv), geom.dtype)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    if dev_err is None:  # a stalled hand-off or unscheduled work is never silent
        dev_err = _default_err(x.device)
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace: must be a contiguous device tensor")
    g = geom.c_struct()
    nbytes = workspace.numel() * workspace.element_size()
    if ckpt_every:
        cap = N // ckpt_every if ckpt_every > 0 else 0
        if ckpt is None and cap == 0:
            ck_bytes = 0
        else:
            if (ckpt is None or not ckpt.is_cuda or ckpt.dtype != torch.float32 or not ckpt.is_contiguous()
                    or ckpt.dim() != 4 or tuple(ckpt.shape[1:]) != (Hv, dv, geom.d_k)):
                raise ValueError(f"ckpt: need a contiguous float32 device tensor [n][{Hv}][{dv}][{geom.d_k}]")
            ck_bytes = ckpt.numel() * 4
        _check(lib().gdn_prefill_chunked_ckpt(ctypes.byref(g), _ptr(pool.state), _ptr(pool.conv_state),
                                              _ptr(pool.conv_pos), _ptr(x), _ptr(a), _ptr(b), _ptr(conv_w),
                                              _ptr(cu_seqlens), _ptr(slot), _ptr(has_init), S, N, CHUNK,
                                              _ptr(workspace), nbytes, _ptr(o), int(ckpt_every), _ptr(ckpt),
                                              ck_bytes, _ptr(dev_err), _stream(stream)))
        return
    _check(lib().gdn_prefill_chunked(ctypes.byref(g), _ptr(pool.state), _ptr(pool.conv_state),
                                     _ptr(pool.conv_pos), _ptr(x), _ptr(a), _ptr(b), _ptr(conv_w),
                                     _ptr(cu_seqlens), _ptr(slot), _ptr(has_init), S, N, CHUNK,
                                     _ptr(workspace), nbytes, _ptr(o), _ptr(dev_err), _stream(stream)))


def prefill_timing_events(start: Optional[torch.cuda.Event], stop: Optional[torch.cuda.Event]):
    """gdn_prefill_timing_events: this thread's next prefill call records
    ``start`` when its plan kernel completes (its main kernel begins) and
    ``stop`` when its main kernel completes (timing events, recorded once
    before so that they exist), through the kernel launches themselves; both
    None clears it."""
    def handle(ev):
        if ev is None:
            return None
        h = ev.cuda_event
        if not h:
            raise ValueError("prefill_timing_events: the event has no HIP event yet (record it once first)")
        return h
    _check(lib().gdn_prefill_timing_events(handle(start), handle(stop)))


def prefill_chunked_static(geom: Geometry, pool: SlotPool, x, a, b, conv_w, cu_seqlens, slot, has_init, o,
                           dev_err=None, stream=None):
    """gdn_prefill_chunked_static: prefill_chunked with the library's own static
    workspace (no allocation in the call; calls that overlap on one GPU race)."""
    N = x.shape[0]
    S = slot.shape[0]
    C, Hv, dv = geom.conv_channels, geom.n_v_heads, geom.d_v
    _check_pool(geom, pool)
    _need(x, "x", (N, C), geom.dtype)
    _need(a, "a", (N, Hv), geom.dtype)
    _need(b, "b", (N, Hv), geom.dtype)
    _need(conv_w, "conv_w", (C, geom.conv_width), torch.float32, optional=geom.conv_width == 0)
    _need(cu_seqlens, "cu_seqlens", (S + 1,), torch.int32)
    _need(slot, "slot", (S,), torch.int32)
    _need(has_init, "has_init", (S,), torch.int32)
    _need(o, "o", (N, Hv, dv), geom.dtype)
    _need(dev_err, "dev_err", (1,), torch.int32, optional=True)
    if dev_err is None:
        dev_err = _default_err(x.device)
    g = geom.c_struct()
    _check(lib().gdn_prefill_chunked_static(ctypes.byref(g), _ptr(pool.state), _ptr(pool.conv_state),
                                            _ptr(pool.conv_pos), _ptr(x), _ptr(a), _ptr(b), _ptr(conv_w),
                                            _ptr(cu_seqlens), _ptr(slot), _ptr(has_init), S, N, CHUNK,
                                            _ptr(o), _ptr(dev_err), _stream(stream)))


def checkpoint_count(seq_lens, ckpt_every: int) -> int:
    """Checkpoints gdn_prefill_chunked_ckpt writes for these sequence lengths."""
    return sum(int(n) // ckpt_every for n in seq_lens)


__all__ = [
    "Geometry", "GdnGeometry", "GdnError", "SlotPool", "lib", "conv_state_step", "decode_step", "verify_k",
    "rollback", "verify_k_slots", "commit_slots", "prefill_chunked", "prefill_chunked_static", "prefill_workspace_bytes", "alloc_prefill_workspace",
    "checkpoint_count", "POS_ONE", "CHUNK",
    "DEV_OK", "DEV_BAD_SLOT", "DEV_BAD_ACCEPTED", "DEV_BAD_SEQLENS", "DEV_WAIT_TIMEOUT", "DEV_BAD_K",
    "DEV_INCOMPLETE", "device_error",
]
