"""The C ABI on the host (no GPU needed): the library loads, exports every
function include/gdn.h declares, validates geometries and refuses bad
arguments with a message naming the argument, the value and the requirement
-- before anything would be launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_delta_amd as m
    if not os.path.exists(m.LIB_PATH):
        from gated_deltanet_delta_amd import build
        build.build()
    m.lib()
    return m


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdn_conv_state_step", "gdn_decode_step", "gdn_prefill_chunked", "gdn_prefill_chunked_ckpt",
              "gdn_verify_k", "gdn_rollback"):
        assert n in names


def test_every_declared_symbol_is_exported(gdn):
    L = gdn.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def _geom(gdn, **kw):
    return gdn.Geometry(**kw).c_struct()


def _check(gdn, g):
    buf = ctypes.create_string_buffer(256)
    st = gdn.lib().gdn_check_geometry(ctypes.byref(g), buf, 256)
    return st, buf.value.decode()


def test_valid_geometries(gdn):
    assert _check(gdn, _geom(gdn))[0] == 0
    tiny = _geom(gdn, n_k_heads=1, n_v_heads=1, d_k=16, d_v=16, conv_width=0, n_slots=1, l2norm_qk=False)
    tiny.dtype_in = tiny.dtype_out = gdn.GDN_F32
    assert _check(gdn, tiny)[0] == 0


@pytest.mark.parametrize("field,value,status,needle", [
    ("n_v_heads", 47, 3, "n_v_heads: 47, required: a multiple of n_k_heads = 16"),
    ("conv_channels", 10000, 3, "conv_channels: 10000, required: 2*n_k_heads*d_k + n_v_heads*d_v = 10240"),
    ("conv_ring", 6, 3, "conv_ring: 6, required: a power of two >= conv_width-1+max_draft = 7"),
    ("conv_ring", 4, 3, "conv_ring: 4"),
    ("conv_width", 5, 3, "conv_width: 5, required: 0..4"),
    ("max_draft", 0, 3, "max_draft: 0"),
    ("n_slots", 0, 3, "n_slots: 0"),
    ("dtype_in", 7, 3, "dtype_in: 7"),
    ("flags", 6, 3, "flags: 0x6"),
])
def test_geometry_refusals_name_found_and_required(gdn, field, value, status, needle):
    g = _geom(gdn)
    setattr(g, field, value)
    st, msg = _check(gdn, g)
    assert st == status and needle in msg, msg


def test_unsupported_sizes_are_refused_not_emulated(gdn):
    g = _geom(gdn, d_k=96, d_v=96)
    st, msg = _check(gdn, g)
    assert st == 4 and "d_k: 96" in msg
    g = _geom(gdn, d_k=128, d_v=64)
    st, msg = _check(gdn, g)
    assert st == 4 and "d_v: 64" in msg
    g = _geom(gdn, n_k_heads=1, n_v_heads=16)
    st, msg = _check(gdn, g)
    assert st == 4 and "n_v_heads/n_k_heads: 16" in msg


def test_workspace_size(gdn):
    """The workspace is a ring of 16 chunk slots of packed operands plus small
    tables: its size does not grow with the number of tokens."""
    g = _geom(gdn)
    L = gdn.lib()
    n1 = L.gdn_prefill_workspace_bytes(ctypes.byref(g), 8192, 1)
    n2 = L.gdn_prefill_workspace_bytes(ctypes.byref(g), 101304, 4)
    n3 = L.gdn_prefill_workspace_bytes(ctypes.byref(g), 1 << 20, 8)
    assert n1 > 0 and n2 == n1 and n3 == n1
    # per (chunk slot, k-head): Q, K and K^T (64 x 128 bf16 each); per v-head of
    # the group: T diag(beta) and P (6 lower-triangle tiles of 16 x 32 each), a
    # 1 KB gate tile and V (64 x 128 bf16)
    per_item = 3 * 64 * 128 * 2 + 3 * (2 * 6 * 1024 + 1024 + 64 * 128 * 2)
    assert abs(n1 - 16 * 16 * per_item) < 256 * 1024
    # a call with fewer chunks than ring slots needs only as many slots
    n4 = L.gdn_prefill_workspace_bytes(ctypes.byref(g), 100, 1)
    assert abs(n4 - 2 * 16 * per_item) < 256 * 1024
    bad = _geom(gdn, n_v_heads=47)
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(bad), 8192, 1) == 0


FAKE = 0x10000  # an aligned address that is never dereferenced: every call below fails validation first


def _p(v=FAKE):
    return ctypes.c_void_p(v)


def test_decode_refusals(gdn):
    L = gdn.lib()
    g = _geom(gdn)
    args = lambda **o: [ctypes.byref(g)] + [o.get(n, _p()) for n in  # noqa: E731
                                            ("state", "conv_state", "conv_pos", "x", "a", "b", "conv_w", "slot")] \
        + [o.get("batch", 4), o.get("o", _p()), None, None]
    assert L.gdn_decode_step(*args(batch=0)) == 5
    assert "batch: 0, required: 1..n_slots = 8" in L.gdn_last_error().decode()
    assert L.gdn_decode_step(*args(batch=9)) == 5
    assert L.gdn_decode_step(*args(state=None)) == 1
    assert "state: NULL" in L.gdn_last_error().decode()
    assert L.gdn_decode_step(*args(x=_p(FAKE + 2))) == 2
    assert "x: address" in L.gdn_last_error().decode() and "16-byte aligned" in L.gdn_last_error().decode()
    assert L.gdn_decode_step(*args(conv_w=None)) == 1
    g.n_v_heads = 47
    assert L.gdn_decode_step(*args()) == 3


def test_verify_and_rollback_refusals(gdn):
    L = gdn.lib()
    g = _geom(gdn)
    va = lambda k: [ctypes.byref(g)] + [_p()] * 7 + [_p(), 4, k, _p(), _p(), None, None]  # noqa: E731
    assert L.gdn_verify_k(*va(0)) == 5
    assert L.gdn_verify_k(*va(5)) == 5
    assert "k: 5, required: 1..max_draft = 4" in L.gdn_last_error().decode()
    rb = [ctypes.byref(g), _p(), _p(), _p(), _p(), None, 4, 4, None, None]
    assert L.gdn_rollback(*rb) == 1
    assert "accepted: NULL" in L.gdn_last_error().decode()


def test_prefill_refusals(gdn):
    L = gdn.lib()
    g = _geom(gdn)
    need = L.gdn_prefill_workspace_bytes(ctypes.byref(g), 8192, 1)

    def call(chunk=64, ws=need, n_seqs=1, n_tokens=8192, cu=_p()):
        return L.gdn_prefill_chunked(ctypes.byref(g), _p(), _p(), _p(), _p(), _p(), _p(), _p(), cu, _p(), _p(),
                                     n_seqs, n_tokens, chunk, _p(), ws, _p(), None, None)
    assert call(chunk=128) == 4
    assert "chunk: 128, supported by this library: 64" in L.gdn_last_error().decode()
    assert call(ws=need - 1) == 6
    assert f"required: >= {need}" in L.gdn_last_error().decode()
    assert call(n_seqs=9) == 5
    assert call(n_tokens=-1) == 5
    assert call(cu=None) == 1
    g.dtype_in = g.dtype_out = gdn.GDN_F32
    assert call() == 4
    assert "d_k: 128 with dtype_in GDN_F32" in L.gdn_last_error().decode()


def test_prefill_static_refusals(gdn):
    """The prefill without a workspace refuses, before touching any GPU, a call
    whose hand-off buffers would not fit the library's static workspace."""
    L = gdn.lib()
    g = _geom(gdn, n_k_heads=64, n_v_heads=192)
    need = L.gdn_prefill_workspace_bytes(ctypes.byref(g), 8192, 1)
    cap = 64 << 20
    assert need > cap

    def call(n_tokens=8192):
        return L.gdn_prefill_chunked_static(ctypes.byref(g), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(),
                                            _p(), 1, n_tokens, 64, _p(), None, None)
    assert call() == 6
    msg = L.gdn_last_error().decode()
    assert f"needs {need} bytes, the static workspace holds {cap}" in msg
    g.n_v_heads = 100  # not a multiple of n_k_heads: the geometry is refused first
    assert call() == 3


def test_prefill_timing_events_requests(gdn):
    """The kernel-timing request takes both events or neither, and the next
    prefill call consumes it even when that call is refused before any launch
    (the handles here are never used: no call below passes validation)."""
    L = gdn.lib()
    assert L.gdn_prefill_timing_events(_p(), None) == 1  # GDN_ERR_NULL
    assert "stop is null" in L.gdn_last_error().decode()
    assert L.gdn_prefill_timing_events(None, _p()) == 1
    assert L.gdn_prefill_timing_events(_p(), _p()) == 0
    g = _geom(gdn, n_k_heads=64, n_v_heads=192)
    assert L.gdn_prefill_chunked_static(ctypes.byref(g), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(),
                                        _p(), 1, 8192, 64, _p(), None, None) == 6
    assert L.gdn_prefill_timing_events(None, None) == 0


def test_prefill_checkpoint_refusals(gdn):
    L = gdn.lib()
    g = _geom(gdn)
    need = L.gdn_prefill_workspace_bytes(ctypes.byref(g), 8192, 1)
    per = g.n_v_heads * g.d_v * g.d_k * 4

    def call(every=512, ck=_p(), ck_bytes=16 * per, n_tokens=8192):
        return L.gdn_prefill_chunked_ckpt(ctypes.byref(g), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(),
                                          _p(), 1, n_tokens, 64, _p(), need, _p(), every, ck, ck_bytes, None, None)
    for bad in (0, -64):
        assert call(every=bad) == 5
        assert f"ckpt_every: {bad}, required: > 0" in L.gdn_last_error().decode()
    assert call(ck_bytes=16 * per - 1) == 5
    assert f"required: >= {16 * per} (16 checkpoints of {per} bytes)" in L.gdn_last_error().decode()
    assert call(ck=None) == 1
    assert "ckpt: NULL" in L.gdn_last_error().decode()
    assert call(ck=ctypes.c_void_p(4096 + 8)) == 2
    # fewer tokens than one block: no checkpoint can be due, so no buffer is needed
    # (the call stops at the next missing pointer, the state)
    st = L.gdn_prefill_chunked_ckpt(ctypes.byref(g), None, _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(),
                                    1, 500, 64, _p(), need, _p(), 512, None, 0, None, None)
    assert st == 1 and "state: NULL" in L.gdn_last_error().decode()


def test_verify_slots_and_commit_refusals(gdn):
    L = gdn.lib()
    g = _geom(gdn, n_slots=20)
    va = lambda batch, k, ss=_p(): [ctypes.byref(g)] + [_p()] * 8 + [batch, k, None, ss, _p(), None, None]  # noqa: E731
    assert L.gdn_verify_k_slots(*va(4, 5)) == 5
    assert "k: 5, required: 1..max_draft = 4" in L.gdn_last_error().decode()
    g.n_slots = 19
    assert L.gdn_verify_k_slots(*va(4, 4)) == 5
    assert "batch * (k + 1): 20, required: <= n_slots = 19" in L.gdn_last_error().decode()
    g.n_slots = 20
    assert L.gdn_verify_k_slots(*va(4, 4, None)) == 1
    assert "snap_slot: NULL" in L.gdn_last_error().decode()
    cm = [ctypes.byref(g), _p(), None, _p(), _p(), 4, 4, None, None, None]
    assert L.gdn_commit_slots(*cm) == 1
    assert "next_slot: NULL" in L.gdn_last_error().decode()
    cm = [ctypes.byref(g), _p(), None, _p(), _p(), 0, 4, _p(), None, None]
    assert L.gdn_commit_slots(*cm) == 5
    # a misaligned per-row count array is refused like any other pointer
    va_k = [ctypes.byref(g)] + [_p()] * 8 + [4, 4, ctypes.c_void_p(0x10000 + 2), _p(), _p(), None, None]
    assert L.gdn_verify_k_slots(*va_k) == 2
    assert "k_row: address" in L.gdn_last_error().decode()


def test_norm_without_conv_refused(gdn):
    """The L2 norm of q and k belongs to the conv front end: without it x holds
    q | k | v as the rule uses them, and asking for the norm is refused."""
    st, msg = _check(gdn, _geom(gdn, conv_width=0))
    assert st == 3 and "GDN_FLAG_L2NORM_QK with conv_width: 0" in msg


def test_conv_step_refusals(gdn):
    L = gdn.lib()
    g = _geom(gdn, conv_width=0, l2norm_qk=False)
    assert L.gdn_conv_state_step(ctypes.byref(g), _p(), _p(), _p(), _p(), _p(), 4, _p(), None, None) == 3
    assert "conv_width: 0" in L.gdn_last_error().decode()


def test_abi_version_matches_the_header(gdn):
    src = open(HEADER).read()
    want = int(re.search(r"#define GDN_ABI_VERSION (\d+)", src).group(1))
    assert gdn.lib().gdn_abi_version() == want == gdn.ABI_VERSION


def test_plain_c_caller(gdn, tmp_path):
    """The header compiles as C99 and a C program links the library and uses
    its host-side entry points (no GPU work)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(gdn.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-lgdn",
                    "-Wl,-rpath," + libdir, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c abi ok" in r.stdout


def test_status_strings(gdn):
    L = gdn.lib()
    assert L.gdn_status_string(0) == b"GDN_OK"
    assert L.gdn_status_string(6) == b"GDN_ERR_WORKSPACE"
    assert b"gfx950" in L.gdn_version()


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import gated_deltanet_delta_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        m.lib()


def test_debug_library_builds_the_same_abi(gdn):
    """libgdn_debug.so (the C ABI built with GDN_DEBUG_CHECKS, which checks a
    call's slot ids on the device) exports every declared symbol of the same
    ABI version and says so in its version string."""
    import os
    path = os.path.join(os.path.dirname(gdn.LIB_PATH), "libgdn_debug.so")
    L = ctypes.CDLL(path)
    assert [n for n in declared_functions() if not hasattr(L, n)] == []
    L.gdn_version.restype = ctypes.c_char_p
    L.gdn_abi_version.restype = ctypes.c_int32
    assert b"debug checks" in L.gdn_version() and b"debug" not in gdn.lib().gdn_version()
    assert L.gdn_abi_version() == gdn.ABI_VERSION
