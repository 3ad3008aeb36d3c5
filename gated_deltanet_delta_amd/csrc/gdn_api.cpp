// C ABI of the GDN library: argument validation and dispatch to the kernel
// launchers.  Host code only; nothing here touches the GPU except the
// launches themselves, which are asynchronous on the caller's stream.
//
// Every refusal names the argument, the value found and the value required
// ("Chapter 6: engine startup and memory plan", section 6.2), and no error is
// swallowed: a launch the runtime refuses is returned as GDN_ERR_LAUNCH with
// the runtime's code ("Forge", entry of 27 August, on a scheduler error that
// went unreported).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

// Debug builds check that a call's slot ids are distinct before its kernels.
#ifdef GDN_DEBUG_CHECKS
#define GDN_DEBUG_DISTINCT(name, a, na, b, nb, kb, k_row)                                               \
  do {                                                                                                 \
    const int e_ = gdn::launch_check_distinct(a, na, b, nb, kb, k_row, dev_err, stream);               \
    if (e_ != 0) return fail(GDN_ERR_LAUNCH, "%s: HIP launch of the slot check failed with error %d", name, e_); \
  } while (0)
#else
#define GDN_DEBUG_DISTINCT(name, a, na, b, nb, kb, k_row) \
  do {                                                  \
  } while (0)
#endif
// kernel-timing events of this thread's next prefill call (gdn_prefill_timing_events)
thread_local void* g_prefill_ev[2] = {nullptr, nullptr};
struct PrefillEvents {
  void* start;
  void* stop;
};
// A pending timing request, taken by the prefill call that begins now.
PrefillEvents take_prefill_events() {
  const PrefillEvents ev{g_prefill_ev[0], g_prefill_ev[1]};
  g_prefill_ev[0] = g_prefill_ev[1] = nullptr;
  return ev;
}

gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gdn_status ok() {
  g_last_error.clear();
  return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define GDN_NEED_PTR(p, name)                                                     \
  do {                                                                            \
    if (!(p)) return fail(GDN_ERR_NULL, "%s: NULL, required: a device pointer", name); \
    if (!aligned16(p))                                                            \
      return fail(GDN_ERR_ALIGN, "%s: address %p, required: 16-byte aligned", name, \
                  static_cast<const void*>(p));                                  \
  } while (0)

#define GDN_NEED_PTR4(p, name)                                                    \
  do {                                                                            \
    if (!(p)) return fail(GDN_ERR_NULL, "%s: NULL, required: a device pointer", name); \
    if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0)                               \
      return fail(GDN_ERR_ALIGN, "%s: address %p, required: 4-byte aligned", name, \
                  static_cast<const void*>(p));                                  \
  } while (0)

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// Workgroups one decode call puts on one slot; the position shares must
// each be at least one unit.
int step_wgs_per_slot(const gdn_geometry& g) { return gdn::decode_wgs_per_slot(g.d_k, g.n_v_heads); }

gdn_status check_geometry(const gdn_geometry* g) {
  if (!g) return fail(GDN_ERR_NULL, "geometry: NULL, required: a gdn_geometry");
  if (g->n_k_heads < 1) return fail(GDN_ERR_GEOMETRY, "n_k_heads: %d, required: >= 1", g->n_k_heads);
  if (g->n_v_heads < 1) return fail(GDN_ERR_GEOMETRY, "n_v_heads: %d, required: >= 1", g->n_v_heads);
  if (g->n_v_heads % g->n_k_heads != 0)
    return fail(GDN_ERR_GEOMETRY, "n_v_heads: %d, required: a multiple of n_k_heads = %d", g->n_v_heads,
                g->n_k_heads);
  if (g->d_k < 1 || g->d_v < 1)
    return fail(GDN_ERR_GEOMETRY, "d_k, d_v: %d, %d, required: >= 1", g->d_k, g->d_v);
  if (g->conv_width < 0 || g->conv_width > 4)
    return fail(GDN_ERR_GEOMETRY, "conv_width: %d, required: 0..4", g->conv_width);
  const long long chan = 2LL * g->n_k_heads * g->d_k + 1LL * g->n_v_heads * g->d_v;
  if (g->conv_channels != chan)
    return fail(GDN_ERR_GEOMETRY, "conv_channels: %d, required: 2*n_k_heads*d_k + n_v_heads*d_v = %lld",
                g->conv_channels, chan);
  if (g->max_draft < 1 || g->max_draft > 16)
    return fail(GDN_ERR_GEOMETRY, "max_draft: %d, required: 1..16", g->max_draft);
  if (g->conv_width > 0) {
    const int need = g->conv_width - 1 + g->max_draft;
    if (!pow2(g->conv_ring) || g->conv_ring < need)
      return fail(GDN_ERR_GEOMETRY,
                  "conv_ring: %d, required: a power of two >= conv_width-1+max_draft = %d", g->conv_ring,
                  need);
    if (g->conv_ring > (1 << 16))
      return fail(GDN_ERR_GEOMETRY, "conv_ring: %d, required: <= 65536", g->conv_ring);
  }
  if (g->n_slots < 1) return fail(GDN_ERR_GEOMETRY, "n_slots: %d, required: >= 1", g->n_slots);
  if (g->dtype_in != GDN_F32 && g->dtype_in != GDN_BF16)
    return fail(GDN_ERR_GEOMETRY, "dtype_in: %d, required: GDN_F32 (0) or GDN_BF16 (1)", g->dtype_in);
  if (g->dtype_out != g->dtype_in)
    return fail(GDN_ERR_UNSUPPORTED, "dtype_out: %d, required: equal to dtype_in = %d", g->dtype_out,
                g->dtype_in);
  if (g->flags & ~GDN_FLAG_L2NORM_QK)
    return fail(GDN_ERR_GEOMETRY, "flags: 0x%x, required: a subset of GDN_FLAG_L2NORM_QK (0x1)", g->flags);
  if (g->conv_width == 0 && (g->flags & GDN_FLAG_L2NORM_QK))
    return fail(GDN_ERR_GEOMETRY,
                "flags: GDN_FLAG_L2NORM_QK with conv_width: 0, required: no flags (without the conv front end "
                "x holds q | k | v exactly as the rule uses them)");
  if (!std::isfinite(g->q_scale)) return fail(GDN_ERR_GEOMETRY, "q_scale: %g, required: finite", g->q_scale);
  if (!std::isfinite(g->l2_eps) || g->l2_eps < 0.f)
    return fail(GDN_ERR_GEOMETRY, "l2_eps: %g, required: finite and >= 0", g->l2_eps);
  if (g->conv_width != 0 && g->conv_width != 4)
    return fail(GDN_ERR_UNSUPPORTED, "conv_width: %d, supported by this library: 0 or 4", g->conv_width);
  if (g->d_k != g->d_v)
    return fail(GDN_ERR_UNSUPPORTED, "d_v: %d, supported by this library: equal to d_k = %d", g->d_v, g->d_k);
  if (g->d_k != 16 && g->d_k != 32 && g->d_k != 64 && g->d_k != 128)
    return fail(GDN_ERR_UNSUPPORTED, "d_k: %d, supported by this library: 16, 32, 64 or 128", g->d_k);
  if (g->n_v_heads / g->n_k_heads > 8)
    return fail(GDN_ERR_UNSUPPORTED, "n_v_heads/n_k_heads: %d, supported by this library: <= 8",
                g->n_v_heads / g->n_k_heads);
  if (step_wgs_per_slot(*g) > (1 << 16))
    return fail(GDN_ERR_UNSUPPORTED, "n_v_heads: %d, supported by this library: at most %d workgroups per slot",
                g->n_v_heads, 1 << 16);
  return ok();
}

gdn::StepArgs step_args(const gdn_geometry* g) {
  gdn::StepArgs a{};
  a.Hk = g->n_k_heads;
  a.Hv = g->n_v_heads;
  a.D = g->d_k;
  a.C = g->conv_channels;
  a.W = g->conv_width;
  a.R = g->conv_ring;
  a.n_slots = g->n_slots;
  a.flags = g->flags;
  a.q_scale = g->q_scale;
  a.l2_eps = g->l2_eps;
  return a;
}

gdn_status launched(int err, const char* what) {
  if (err != 0) return fail(GDN_ERR_LAUNCH, "%s: HIP launch failed with error %d", what, err);
  return ok();
}

gdn_status check_batch(int32_t batch, const gdn_geometry* g) {
  if (batch < 1 || batch > g->n_slots)
    return fail(GDN_ERR_RANGE, "batch: %d, required: 1..n_slots = %d", batch, g->n_slots);
  return GDN_OK;
}

}  // namespace

static gdn_status prefill_call(const gdn_geometry* g, float* state, float* conv_state, int32_t* conv_pos,
                               const void* x, const void* a_in, const void* b_in, const float* conv_w,
                               const int32_t* cu_seqlens, const int32_t* slot, const int32_t* has_init,
                               int32_t n_seqs, int32_t n_tokens, int32_t chunk, void* workspace,
                               size_t workspace_bytes, void* o, int32_t ckpt_every, float* ckpt,
                               size_t ckpt_bytes, int32_t* dev_err, void* stream, const char* name,
                               const PrefillEvents& ev);

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN";
    case GDN_ERR_GEOMETRY: return "GDN_ERR_GEOMETRY";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_RANGE: return "GDN_ERR_RANGE";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH";
  }
  return "GDN_ERR_UNKNOWN";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

gdn_status gdn_prefill_timing_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(GDN_ERR_NULL, "gdn_prefill_timing_events: %s is null, required: both events or neither",
                start == nullptr ? "start" : "stop");
  g_prefill_ev[0] = start;
  g_prefill_ev[1] = stop;
  return GDN_OK;
}

#ifdef GDN_DEBUG_CHECKS
const char* gdn_version(void) { return "gdn-mi355x 0.2 (gfx950, debug checks)"; }
#else
const char* gdn_version(void) { return "gdn-mi355x 0.2 (gfx950)"; }
#endif

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_check_geometry(const gdn_geometry* g, char* msg, size_t msg_len) {
  const gdn_status s = check_geometry(g);
  if (msg && msg_len) {
    std::strncpy(msg, g_last_error.c_str(), msg_len - 1);
    msg[msg_len - 1] = '\0';
  }
  return s;
}

size_t gdn_prefill_workspace_bytes(const gdn_geometry* g, int32_t n_tokens, int32_t n_seqs) {
  if (check_geometry(g) != GDN_OK || n_tokens < 0 || n_seqs < 1) return 0;
  return gdn::prefill_layout(g->n_k_heads, g->n_v_heads, g->d_k, g->dtype_in == GDN_BF16, n_tokens, n_seqs).total;
}

gdn_status gdn_conv_state_step(const gdn_geometry* g, float* conv_state, int32_t* conv_pos, const void* x,
                               const float* conv_w, const int32_t* slot, int32_t batch, void* y,
                               int32_t* dev_err, void* stream) {
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  if (g->conv_width < 1)
    return fail(GDN_ERR_GEOMETRY, "conv_width: %d, required: >= 1 for gdn_conv_state_step", g->conv_width);
  if ((s = check_batch(batch, g)) != GDN_OK) return s;
  GDN_NEED_PTR(conv_state, "conv_state");
  GDN_NEED_PTR4(conv_pos, "conv_pos");
  GDN_NEED_PTR(x, "x");
  GDN_NEED_PTR(conv_w, "conv_w");
  GDN_NEED_PTR4(slot, "slot");
  GDN_NEED_PTR(y, "y");
  gdn::StepArgs a = step_args(g);
  a.conv_state = conv_state;
  a.conv_pos = conv_pos;
  a.x = x;
  a.conv_w = conv_w;
  a.slot = slot;
  a.o = y;
  a.dev_err = dev_err;
  a.batch = batch;
  a.k = 1;
  GDN_DEBUG_DISTINCT("gdn_conv_state_step", slot, batch, nullptr, 0, 0, nullptr);
  return launched(gdn::launch_conv_step(a, g->dtype_in == GDN_BF16, stream), "gdn_conv_state_step");
}

gdn_status gdn_decode_step(const gdn_geometry* g, float* state, float* conv_state, int32_t* conv_pos,
                           const void* x, const void* a_in, const void* b_in, const float* conv_w,
                           const int32_t* slot, int32_t batch, void* o, int32_t* dev_err, void* stream) {
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  if ((s = check_batch(batch, g)) != GDN_OK) return s;
  GDN_NEED_PTR(state, "state");
  if (g->conv_width > 0) {
    GDN_NEED_PTR(conv_state, "conv_state");
    GDN_NEED_PTR4(conv_pos, "conv_pos");
    GDN_NEED_PTR(conv_w, "conv_w");
  }
  GDN_NEED_PTR(x, "x");
  GDN_NEED_PTR(a_in, "a");
  GDN_NEED_PTR(b_in, "b");
  GDN_NEED_PTR4(slot, "slot");
  GDN_NEED_PTR(o, "o");
  gdn::StepArgs a = step_args(g);
  a.state = state;
  a.conv_state = conv_state;
  a.conv_pos = conv_pos;
  a.x = x;
  a.a = a_in;
  a.b = b_in;
  a.conv_w = conv_w;
  a.slot = slot;
  a.o = o;
  a.dev_err = dev_err;
  a.batch = batch;
  a.k = 1;
  GDN_DEBUG_DISTINCT("gdn_decode_step", slot, batch, nullptr, 0, 0, nullptr);
  return launched(gdn::launch_decode(a, g->dtype_in == GDN_BF16, stream), "gdn_decode_step");
}

gdn_status gdn_verify_k(const gdn_geometry* g, const float* state, float* conv_state, const int32_t* conv_pos,
                        const void* x, const void* a_in, const void* b_in, const float* conv_w,
                        const int32_t* slot, int32_t batch, int32_t k, float* snap, void* o, int32_t* dev_err,
                        void* stream) {
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  if ((s = check_batch(batch, g)) != GDN_OK) return s;
  if (k < 1 || k > g->max_draft)
    return fail(GDN_ERR_RANGE, "k: %d, required: 1..max_draft = %d", k, g->max_draft);
  GDN_NEED_PTR(state, "state");
  if (g->conv_width > 0) {
    GDN_NEED_PTR(conv_state, "conv_state");
    GDN_NEED_PTR4(conv_pos, "conv_pos");
    GDN_NEED_PTR(conv_w, "conv_w");
  }
  GDN_NEED_PTR(x, "x");
  GDN_NEED_PTR(a_in, "a");
  GDN_NEED_PTR(b_in, "b");
  GDN_NEED_PTR4(slot, "slot");
  GDN_NEED_PTR(snap, "snap");
  GDN_NEED_PTR(o, "o");
  gdn::StepArgs a = step_args(g);
  a.state = const_cast<float*>(state);  // read only in verify
  a.conv_state = conv_state;
  a.conv_pos = const_cast<int32_t*>(conv_pos);
  a.x = x;
  a.a = a_in;
  a.b = b_in;
  a.conv_w = conv_w;
  a.slot = slot;
  a.o = o;
  a.snap = snap;
  a.dev_err = dev_err;
  a.batch = batch;
  a.k = k;
  GDN_DEBUG_DISTINCT("gdn_verify_k", slot, batch, nullptr, 0, 0, nullptr);
  return launched(gdn::launch_verify(a, g->dtype_in == GDN_BF16, stream), "gdn_verify_k");
}

gdn_status gdn_verify_k_slots(const gdn_geometry* g, float* state, float* conv_state, int32_t* conv_pos,
                              const void* x, const void* a_in, const void* b_in, const float* conv_w,
                              const int32_t* slot, int32_t batch, int32_t k, const int32_t* k_row,
                              const int32_t* snap_slot, void* o, int32_t* dev_err, void* stream) {
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  if ((s = check_batch(batch, g)) != GDN_OK) return s;
  if (k < 1 || k > g->max_draft)
    return fail(GDN_ERR_RANGE, "k: %d, required: 1..max_draft = %d", k, g->max_draft);
  if (static_cast<int64_t>(batch) * (k + 1) > g->n_slots)
    return fail(GDN_ERR_RANGE, "batch * (k + 1): %lld, required: <= n_slots = %d (rows and snapshots need distinct slots)",
                static_cast<long long>(batch) * (k + 1), g->n_slots);
  GDN_NEED_PTR(state, "state");
  if (g->conv_width > 0) {
    GDN_NEED_PTR(conv_state, "conv_state");
    GDN_NEED_PTR4(conv_pos, "conv_pos");
    GDN_NEED_PTR(conv_w, "conv_w");
  }
  GDN_NEED_PTR(x, "x");
  GDN_NEED_PTR(a_in, "a");
  GDN_NEED_PTR(b_in, "b");
  GDN_NEED_PTR4(slot, "slot");
  GDN_NEED_PTR4(snap_slot, "snap_slot");
  GDN_NEED_PTR(o, "o");
  gdn::StepArgs a = step_args(g);
  a.state = state;
  a.conv_state = conv_state;
  a.conv_pos = conv_pos;
  a.x = x;
  a.a = a_in;
  a.b = b_in;
  a.conv_w = conv_w;
  a.slot = slot;
  a.snap_slot = snap_slot;
  if (k_row) GDN_NEED_PTR4(k_row, "k_row");
  a.k_row = k_row;
  a.o = o;
  a.dev_err = dev_err;
  a.batch = batch;
  a.k = k;
  GDN_DEBUG_DISTINCT("gdn_verify_k_slots", slot, batch, snap_slot, batch, k, k_row);
  return launched(gdn::launch_verify(a, g->dtype_in == GDN_BF16, stream), "gdn_verify_k_slots");
}

gdn_status gdn_commit_slots(const gdn_geometry* g, const int32_t* slot, const int32_t* k_row,
                            const int32_t* snap_slot, const int32_t* accepted, int32_t batch, int32_t k,
                            int32_t* next_slot, int32_t* dev_err, void* stream) {
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  if ((s = check_batch(batch, g)) != GDN_OK) return s;
  if (k < 1 || k > g->max_draft)
    return fail(GDN_ERR_RANGE, "k: %d, required: 1..max_draft = %d", k, g->max_draft);
  GDN_NEED_PTR4(slot, "slot");
  GDN_NEED_PTR4(snap_slot, "snap_slot");
  GDN_NEED_PTR4(accepted, "accepted");
  GDN_NEED_PTR4(next_slot, "next_slot");
  gdn::StepArgs a = step_args(g);
  a.slot = slot;
  a.snap_slot = snap_slot;
  if (k_row) GDN_NEED_PTR4(k_row, "k_row");
  a.k_row = k_row;
  a.accepted = accepted;
  a.next_slot = next_slot;
  a.dev_err = dev_err;
  a.batch = batch;
  a.k = k;
  return launched(gdn::launch_commit_slots(a, stream), "gdn_commit_slots");
}

gdn_status gdn_rollback(const gdn_geometry* g, float* state, int32_t* conv_pos, const float* snap,
                        const int32_t* slot, const int32_t* accepted, int32_t batch, int32_t k, int32_t* dev_err,
                        void* stream) {
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  if ((s = check_batch(batch, g)) != GDN_OK) return s;
  if (k < 1 || k > g->max_draft)
    return fail(GDN_ERR_RANGE, "k: %d, required: 1..max_draft = %d", k, g->max_draft);
  GDN_NEED_PTR(state, "state");
  if (g->conv_width > 0) GDN_NEED_PTR4(conv_pos, "conv_pos");
  GDN_NEED_PTR(snap, "snap");
  GDN_NEED_PTR4(slot, "slot");
  GDN_NEED_PTR4(accepted, "accepted");
  gdn::StepArgs a = step_args(g);
  a.state = state;
  a.conv_pos = conv_pos;
  a.snap = const_cast<float*>(snap);
  a.slot = slot;
  a.accepted = accepted;
  a.dev_err = dev_err;
  a.batch = batch;
  a.k = k;
  GDN_DEBUG_DISTINCT("gdn_rollback", slot, batch, nullptr, 0, 0, nullptr);
  return launched(gdn::launch_rollback(a, stream), "gdn_rollback");
}

gdn_status gdn_prefill_chunked(const gdn_geometry* g, float* state, float* conv_state, int32_t* conv_pos,
                               const void* x, const void* a_in, const void* b_in, const float* conv_w,
                               const int32_t* cu_seqlens, const int32_t* slot, const int32_t* has_init,
                               int32_t n_seqs, int32_t n_tokens, int32_t chunk, void* workspace,
                               size_t workspace_bytes, void* o, int32_t* dev_err, void* stream) {
  const PrefillEvents ev = take_prefill_events();
  return prefill_call(g, state, conv_state, conv_pos, x, a_in, b_in, conv_w, cu_seqlens, slot, has_init, n_seqs,
                      n_tokens, chunk, workspace, workspace_bytes, o, 0, nullptr, 0, dev_err, stream,
                      "gdn_prefill_chunked", ev);
}

gdn_status gdn_prefill_chunked_static(const gdn_geometry* g, float* state, float* conv_state, int32_t* conv_pos,
                                      const void* x, const void* a_in, const void* b_in, const float* conv_w,
                                      const int32_t* cu_seqlens, const int32_t* slot, const int32_t* has_init,
                                      int32_t n_seqs, int32_t n_tokens, int32_t chunk, void* o, int32_t* dev_err,
                                      void* stream) {
  const char* name = "gdn_prefill_chunked_static";
  const PrefillEvents ev = take_prefill_events();
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  const size_t need = gdn_prefill_workspace_bytes(g, n_tokens, n_seqs);
  if (need > GDN_PREFILL_STATIC_WORKSPACE_BYTES)
    return fail(GDN_ERR_WORKSPACE,
                "workspace: this call needs %zu bytes, the static workspace holds %zu; call gdn_prefill_chunked "
                "with a workspace of its own",
                need, static_cast<size_t>(GDN_PREFILL_STATIC_WORKSPACE_BYTES));
  void* ws = nullptr;
  const int e = gdn::prefill_static_workspace(stream, &ws);
  if (e != 0) return fail(GDN_ERR_LAUNCH, "%s: static workspace address not available (HIP error %d)", name, e);
  return prefill_call(g, state, conv_state, conv_pos, x, a_in, b_in, conv_w, cu_seqlens, slot, has_init, n_seqs,
                      n_tokens, chunk, ws, GDN_PREFILL_STATIC_WORKSPACE_BYTES, o, 0, nullptr, 0, dev_err, stream,
                      name, ev);
}

gdn_status gdn_prefill_chunked_ckpt(const gdn_geometry* g, float* state, float* conv_state, int32_t* conv_pos,
                                    const void* x, const void* a_in, const void* b_in, const float* conv_w,
                                    const int32_t* cu_seqlens, const int32_t* slot, const int32_t* has_init,
                                    int32_t n_seqs, int32_t n_tokens, int32_t chunk, void* workspace,
                                    size_t workspace_bytes, void* o, int32_t ckpt_every, float* ckpt,
                                    size_t ckpt_bytes, int32_t* dev_err, void* stream) {
  const PrefillEvents ev = take_prefill_events();
  if (ckpt_every <= 0)
    return fail(GDN_ERR_RANGE, "ckpt_every: %d, required: > 0", ckpt_every);
  return prefill_call(g, state, conv_state, conv_pos, x, a_in, b_in, conv_w, cu_seqlens, slot, has_init, n_seqs,
                      n_tokens, chunk, workspace, workspace_bytes, o, ckpt_every, ckpt, ckpt_bytes, dev_err,
                      stream, "gdn_prefill_chunked_ckpt", ev);
}

}  // extern "C"

// Both prefill entry points: checks, then the launch.  ckpt_every == 0: no checkpoints.
static gdn_status prefill_call(const gdn_geometry* g, float* state, float* conv_state, int32_t* conv_pos,
                               const void* x, const void* a_in, const void* b_in, const float* conv_w,
                               const int32_t* cu_seqlens, const int32_t* slot, const int32_t* has_init,
                               int32_t n_seqs, int32_t n_tokens, int32_t chunk, void* workspace,
                               size_t workspace_bytes, void* o, int32_t ckpt_every, float* ckpt,
                               size_t ckpt_bytes, int32_t* dev_err, void* stream, const char* name,
                               const PrefillEvents& ev) {
  gdn_status s = check_geometry(g);
  if (s != GDN_OK) return s;
  if (chunk != gdn::kChunk)
    return fail(GDN_ERR_UNSUPPORTED, "chunk: %d, supported by this library: %d", chunk, gdn::kChunk);
  if (g->dtype_in == GDN_F32 && g->d_k > 64)
    return fail(GDN_ERR_UNSUPPORTED, "d_k: %d with dtype_in GDN_F32, supported by this library for prefill: <= 64",
                g->d_k);
  if (n_seqs < 1 || n_seqs > g->n_slots)
    return fail(GDN_ERR_RANGE, "n_seqs: %d, required: 1..n_slots = %d", n_seqs, g->n_slots);
  if (n_tokens < 0) return fail(GDN_ERR_RANGE, "n_tokens: %d, required: >= 0", n_tokens);
  const size_t need = gdn_prefill_workspace_bytes(g, n_tokens, n_seqs);
  if (workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "workspace_bytes: %zu, required: >= %zu", workspace_bytes, need);
  GDN_NEED_PTR(state, "state");
  if (g->conv_width > 0) {
    GDN_NEED_PTR(conv_state, "conv_state");
    GDN_NEED_PTR4(conv_pos, "conv_pos");
    GDN_NEED_PTR(conv_w, "conv_w");
  }
  if (n_tokens > 0) {
    GDN_NEED_PTR(x, "x");
    GDN_NEED_PTR(a_in, "a");
    GDN_NEED_PTR(b_in, "b");
    GDN_NEED_PTR(o, "o");
  }
  GDN_NEED_PTR4(cu_seqlens, "cu_seqlens");
  GDN_NEED_PTR4(slot, "slot");
  GDN_NEED_PTR4(has_init, "has_init");
  GDN_NEED_PTR(workspace, "workspace");
  gdn::PrefillArgs a{};
  a.state = state;
  a.conv_state = conv_state;
  a.conv_pos = conv_pos;
  a.x = x;
  a.a = a_in;
  a.b = b_in;
  a.conv_w = conv_w;
  a.cu_seqlens = cu_seqlens;
  a.slot = slot;
  a.has_init = has_init;
  a.o = o;
  a.dev_err = dev_err;
  a.workspace = workspace;
  a.n_seqs = n_seqs;
  a.n_tokens = n_tokens;
  a.max_chunks = gdn::prefill_max_chunks(n_tokens, n_seqs);
  a.Hk = g->n_k_heads;
  a.Hv = g->n_v_heads;
  a.D = g->d_k;
  a.C = g->conv_channels;
  a.W = g->conv_width;
  a.R = g->conv_ring;
  a.n_slots = g->n_slots;
  a.flags = g->flags;
  a.q_scale = g->q_scale;
  a.l2_eps = g->l2_eps;
  if (ckpt_every > 0) {
    const size_t n_ckpt = static_cast<size_t>(n_tokens / ckpt_every);
    const size_t per = static_cast<size_t>(g->n_v_heads) * g->d_v * g->d_k * sizeof(float);
    if (ckpt_bytes < n_ckpt * per)
      return fail(GDN_ERR_RANGE, "ckpt_bytes: %zu, required: >= %zu (%zu checkpoints of %zu bytes)", ckpt_bytes,
                  n_ckpt * per, n_ckpt, per);
    if (n_ckpt > 0) GDN_NEED_PTR(ckpt, "ckpt");
    a.ckpt = ckpt;
    a.ckpt_every = ckpt_every;
  }
  GDN_DEBUG_DISTINCT(name, slot, n_seqs, nullptr, 0, 0, nullptr);
  return launched(gdn::launch_prefill(a, g->dtype_in == GDN_BF16, stream, ev.start, ev.stop), name);
}
