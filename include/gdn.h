/*
 * gdn.h -- C ABI of the Gated DeltaNet layer library for AMD MI355X (gfx950).
 *
 * The layer (Gated DeltaNet, arXiv:2412.06464; described in words in
 * "Hybrid transformers under load: where Gated DeltaNet loses to full
 * attention", section 3) keeps a fixed-size fp32 state S (d_v x d_k) per
 * v-head and, for every token,
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = q_scale * S_t q_t,
 *
 * with alpha_t = exp(-softplus(a_t)) and beta_t = sigmoid(b_t) from the raw
 * gate inputs a, b, and q, k, v taken from the projected input x through a
 * causal depthwise conv of width W, SiLU, and an L2 normalisation of q and k
 * (x * (sum x^2 + l2_eps)^-1/2 per k-head).  The conv input channels are
 * ordered q | k | v, each head-major; v-head h reads k-head h / (H_v / H_k).
 *
 * Three paths share one slot pool: a per-token decode step, a chunked
 * (WY/UT-transform) prefill over variable-length sequences, and a k-draft
 * speculative verify that writes a state snapshot after every draft so that
 * rollback is a copy ("Forge: how I wrote my own inference engine and beat
 * llama.cpp", entry of 27 August).
 *
 * Conventions for every call below
 * --------------------------------
 *  - Pointers are DEVICE pointers unless stated otherwise; every buffer is
 *    owned by the caller.  The library never allocates, frees or synchronises
 *    on these calls: work is enqueued on `stream` (a hipStream_t, NULL = the
 *    default stream) and the call returns ("Chapter 6: engine startup and
 *    memory plan", section 6.10: the token path allocates nothing).
 *  - Problems the host can see (bad geometry, null or misaligned pointers,
 *    sizes out of range, small workspace) return a nonzero gdn_status BEFORE
 *    anything is launched; gdn_last_error() then names the argument, the value
 *    found and the value required (same book, section 6.2: a mismatch is
 *    reported with the name, the shape found and the shape required).
 *  - Problems only the device can see (a slot id out of [0, n_slots), an
 *    accepted length out of [0, k], cu_seqlens that are not a valid partition)
 *    are written to *dev_err (if dev_err is not NULL) as the FIRST error code
 *    of the call (later ones do not overwrite it) and the affected row is
 *    skipped: nothing is clamped, nothing is written out of range.
 *  - Buffers read or written by a call must not alias each other (x, a, b,
 *    o, snap, workspace vs state and conv_state).  Slot ids within one call
 *    must be distinct; duplicates give undefined results.  A library built
 *    with GDN_DEBUG_CHECKS (libgdn_debug.so) checks this on the device before
 *    each call's kernels and writes GDN_DEV_DUP_SLOT to *dev_err (calls
 *    without dev_err are not checked); the release library does not.
 *  - Every pointer to float data and every x / o / snap / workspace pointer
 *    must be 16-byte aligned.
 *  - Calls on one stream are ordered; calls that overlap in time on the same
 *    slots race.
 *
 * Layouts (row-major, last index fastest)
 * ---------------------------------------
 *  state      fp32  [n_slots][H_v][d_v][d_k]   slot pool of recurrent states
 *  conv_state fp32  [n_slots][R][C]            conv ring of past inputs x
 *  conv_pos   int32 [n_slots][GDN_POS_STRIDE]  ring position of slot s in
 *                                              conv_pos[s][0], in units of
 *                                              1/GDN_POS_ONE token (below);
 *                                              words 1.. of a row are never
 *                                              read or written
 *  conv_w     fp32  [C][W]                     tap W-1 multiplies the current token
 *  x          dtype_in  [rows][C]              projected input, q | k | v
 *  a, b       dtype_in  [rows][H_v]            raw gate inputs
 *  o          dtype_out [rows][H_v][d_v]
 *
 * The conv ring.  Row (p mod R) of a slot's ring holds the input x of the
 * slot's token number p; the conv window of the next token reads rows
 * p-W+1 .. p-1 (mod R) for the current position p.  conv_pos keeps p scaled
 * by GDN_POS_ONE (65536) so that the many workgroups of one call can each add
 * a fraction of one token without a second counter: readers take
 * p = (uint32_t)conv_pos >> 16.  The ring must hold R >= W-1+max_draft rows
 * (R a power of two) so verify can write its drafts ahead of the committed
 * history without overwriting it.  Zero-initialising a slot's ring and
 * conv_pos gives an all-zero history.  Each slot's position has a 128-byte
 * line of its own (GDN_POS_STRIDE words), so that the position updates of
 * different slots in one call do not contend for one line of the cache.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 7  /* 4: prefill on the caller's stream alone, workspace independent of n_tokens,
                              checkpoints at any block size, GDN_DEV_INCOMPLETE;
                              5: gdn_prefill_chunked_static;
                              6: gdn_prefill_timing_events;
                              7: GDN_DEV_DUP_SLOT (debug builds) */
/* bytes of the library's own prefill workspace, one per GPU (gdn_prefill_chunked_static) */
#define GDN_PREFILL_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
#define GDN_POS_ONE 65536
#define GDN_POS_STRIDE 32 /* int32 words per slot in conv_pos */

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,          /* a required pointer is NULL */
  GDN_ERR_ALIGN = 2,         /* a pointer is not 16-byte aligned */
  GDN_ERR_GEOMETRY = 3,      /* inconsistent gdn_geometry */
  GDN_ERR_UNSUPPORTED = 4,   /* a valid geometry the library has no kernels for */
  GDN_ERR_RANGE = 5,         /* a size argument out of range (batch, k, n_tokens...) */
  GDN_ERR_WORKSPACE = 6,     /* workspace smaller than gdn_prefill_workspace_bytes() */
  GDN_ERR_LAUNCH = 7         /* the HIP runtime refused a launch */
} gdn_status;

/* Device-side error codes written to *dev_err (first one wins). */
#define GDN_DEV_OK 0
#define GDN_DEV_BAD_SLOT 1       /* slot id outside [0, n_slots) */
#define GDN_DEV_BAD_ACCEPTED 2   /* accepted length outside [0, k] */
#define GDN_DEV_BAD_SEQLENS 3    /* cu_seqlens[0] != 0, decreasing, or last != n_tokens */
#define GDN_DEV_WAIT_TIMEOUT 4   /* prefill: a hand-off between its workgroups stalled (bounded wait); outputs invalid */
#define GDN_DEV_BAD_K 5          /* a row's draft count outside [1, k] */
#define GDN_DEV_INCOMPLETE 6     /* prefill: part of the work was never picked up by a workgroup; outputs invalid */
#define GDN_DEV_DUP_SLOT 7       /* two rows of one call name the same slot; written only by a library built with
                                    GDN_DEBUG_CHECKS (libgdn_debug.so), which checks this before each call's kernels */

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

#define GDN_FLAG_L2NORM_QK 1u    /* L2-normalise q and k after the conv front end (requires conv_width > 0) */

/*
 * Geometry of one layer.  Every field is a number some kernel depends on
 * ("Chapter 6: engine startup and memory plan", section 6.2, ModelGeometry:
 * ssm_state_size = 128, ssm_k_heads = 16, ssm_v_heads = 48, ssm_d_conv = 4,
 * ssm_conv_channels = 10240 = 2*128*16 + 128*48).
 */
typedef struct gdn_geometry {
  int32_t n_k_heads;      /* H_k */
  int32_t n_v_heads;      /* H_v, a multiple of H_k */
  int32_t d_k;            /* state columns (ssm_state_size) */
  int32_t d_v;            /* state rows; the library requires d_v == d_k in {16,32,64,128} */
  int32_t conv_width;     /* W in 0..4 (this library: 0 or 4); 0 = no conv and no SiLU: x holds q | k | v */
  int32_t conv_channels;  /* C, must equal 2*H_k*d_k + H_v*d_v */
  int32_t conv_ring;      /* R, power of two >= W-1+max_draft (ignored when W = 0) */
  int32_t max_draft;      /* largest k accepted by gdn_verify_k (1..16) */
  int32_t n_slots;        /* pool size */
  int32_t dtype_in;       /* gdn_dtype of x, a, b */
  int32_t dtype_out;      /* gdn_dtype of o and of gdn_conv_state_step's y; == dtype_in */
  uint32_t flags;         /* GDN_FLAG_* */
  float q_scale;          /* output scale; 1.0 computes o = S q as written */
  float l2_eps;           /* epsilon under the square root of the L2 norm (1e-6) */
} gdn_geometry;

/* Human-readable name of a status code (static storage). */
const char* gdn_status_string(gdn_status s);

/* Message of the last failing call on this host thread ("" if none). */
const char* gdn_last_error(void);

/* Library version string (static storage). */
const char* gdn_version(void);

/* GDN_ABI_VERSION the library was built with; a caller built against another
 * version of this header must not use it. */
int32_t gdn_abi_version(void);

/*
 * Validate a geometry without touching the GPU.  Returns GDN_OK, or an error
 * with a message (also copied into msg when msg != NULL, NUL-terminated,
 * truncated to msg_len) naming the field, the value found and the value
 * required.  GDN_ERR_UNSUPPORTED means consistent but not built here.
 * ("Chapter 6: engine startup and memory plan", section 6.2: the layer's
 * geometry is checked once at start-up, and a refusal states the field, the
 * value found and the value required.)
 */
gdn_status gdn_check_geometry(const gdn_geometry* g, char* msg, size_t msg_len);

/*
 * Workspace bytes gdn_prefill_chunked needs for n_tokens tokens in n_seqs
 * sequences with 64-token chunks (0 when the geometry is invalid).  Host only.
 * The size is bounded independently of n_tokens: chunks pass between the
 * prefill's workgroups through a ring of at most 16 chunk slots (fewer when
 * the call has fewer chunks), plus a table of n_seqs entries and flags.
 * ("Chapter 6: engine startup and memory plan", section 6.10: the memory
 * of the token path is planned up front and bounded.)
 */
size_t gdn_prefill_workspace_bytes(const gdn_geometry* g, int32_t n_tokens, int32_t n_seqs);

/*
 * The conv front end alone, one token per batch row: for every one of the C
 * channels, y = SiLU(causal depthwise conv over the slot's last W-1 inputs
 * and x) (taps oldest first, conv_w [C][W] fp32), then x is appended to the
 * slot's ring and conv_pos advances one token.  No norm, gates or state.
 *   x [batch][C] (dtype_in), y [batch][C] (dtype_out), slot [batch] int32.
 *   1 <= batch <= n_slots; requires conv_width = 4.
 * ("Hybrid transformers under load", section 3: the short causal
 * convolution ahead of the delta rule, whose state between tokens is the last
 * W-1 inputs; "Chapter 6: engine startup and memory plan", section 6.2:
 * ssm_d_conv = 4 over ssm_conv_channels = 10240.)
 */
gdn_status gdn_conv_state_step(const gdn_geometry* g, float* conv_state, int32_t* conv_pos,
                               const void* x, const float* conv_w, const int32_t* slot,
                               int32_t batch, void* y, int32_t* dev_err, void* stream);

/*
 * One decode token per batch row, fused: conv ring + SiLU, L2 norm of q and k,
 * gates, the delta-rule update of the slot's state in place, and the output.
 * Each fp32 state row is read once and written once ("Hybrid transformers
 * under load", section 3: the gated delta rule, one token at a time against
 * a fixed-size state; "Forge", section on the formulas that decide
 * everything: a decode step costs the bytes it moves over the bandwidth).
 *   x [batch][C], a, b [batch][H_v] (dtype_in); o [batch][H_v][d_v] (dtype_out);
 *   slot [batch] int32 (device).  Advances conv_pos of each slot by one token.
 *   1 <= batch <= n_slots.
 */
gdn_status gdn_decode_step(const gdn_geometry* g, float* state, float* conv_state,
                           int32_t* conv_pos, const void* x, const void* a, const void* b,
                           const float* conv_w, const int32_t* slot, int32_t batch, void* o,
                           int32_t* dev_err, void* stream);

/*
 * Chunked prefill of n_seqs sequences packed along the token axis
 * (cu_seqlens [n_seqs+1] int32, device: sequence s is tokens
 * [cu_seqlens[s], cu_seqlens[s+1])).  Sequence s starts from slot[s]'s state
 * and conv history when has_init[s] != 0, from zeros otherwise; its final
 * state and conv history are written back to slot[s] and conv_pos[slot[s]]
 * ends n_s tokens after the start position (0 when has_init[s] == 0).
 * Chunks of `chunk` = 64 tokens never straddle two sequences; the last chunk
 * of a sequence may be partial.  Results equal the token-by-token rule up to
 * rounding (the chunked form is an exact reorganisation).
 *   x [n_tokens][C], a, b [n_tokens][H_v] (dtype_in); o [n_tokens][H_v][d_v];
 *   slot, has_init [n_seqs] int32 (device).
 *   workspace: device, >= gdn_prefill_workspace_bytes(g, n_tokens, n_seqs).
 *   1 <= n_seqs <= n_slots, 0 <= n_tokens.
 * Both kernels of the call (a planning kernel, then one launch that holds
 * the chunk-parallel and the sequential parts as cooperating workgroups) are
 * enqueued on `stream` alone; the call creates no stream or event and keeps
 * no state between calls, so it may be captured into a graph.  Calls that
 * share a workspace must be ordered on one stream.  *dev_err receives
 * GDN_DEV_WAIT_TIMEOUT if a hand-off between the launch's workgroups ever
 * stalls past its bounded wait, or GDN_DEV_INCOMPLETE if part of the work was
 * never taken up (the outputs are then not valid); the launch always ends.
 * (The chunked form: the rule of "Hybrid transformers under load", section
 * 3, reorganised over 64-token chunks; same results up to rounding.)
 */
gdn_status gdn_prefill_chunked(const gdn_geometry* g, float* state, float* conv_state,
                               int32_t* conv_pos, const void* x, const void* a, const void* b,
                               const float* conv_w, const int32_t* cu_seqlens,
                               const int32_t* slot, const int32_t* has_init, int32_t n_seqs,
                               int32_t n_tokens, int32_t chunk, void* workspace,
                               size_t workspace_bytes, void* o, int32_t* dev_err, void* stream);

/*
 * gdn_prefill_chunked for callers that cannot allocate device memory (code
 * under graph capture that may not call the allocator, serving loops and
 * harnesses that forbid allocation): the same computation and results, bit
 * for bit, with no workspace argument.  The hand-off buffers live in a static
 * device array of GDN_PREFILL_STATIC_WORKSPACE_BYTES (64 MiB) that the library
 * holds on each GPU it runs on until the process ends; its address on a GPU
 * is looked up once, on the first call there.  The call allocates nothing.
 * The GPU is the one `stream` belongs to (the current device for the null
 * stream).  All calls on one GPU share the array: calls that overlap in time
 * on one GPU (two streams, two host threads) race and must be ordered, e.g.
 * on one stream; every call clears the flags it uses before its main launch.
 * Errors as gdn_prefill_chunked, with GDN_ERR_WORKSPACE when
 * gdn_prefill_workspace_bytes(g, n_tokens, n_seqs) exceeds the array (the
 * 16 k-head, 48 v-head, d = 128 bf16 geometry needs about 34 MB at any
 * n_tokens) and GDN_ERR_LAUNCH when the array's address cannot be had.
 */
gdn_status gdn_prefill_chunked_static(const gdn_geometry* g, float* state, float* conv_state,
                                      int32_t* conv_pos, const void* x, const void* a, const void* b,
                                      const float* conv_w, const int32_t* cu_seqlens,
                                      const int32_t* slot, const int32_t* has_init, int32_t n_seqs,
                                      int32_t n_tokens, int32_t chunk, void* o, int32_t* dev_err,
                                      void* stream);

/*
 * gdn_prefill_chunked that also writes state checkpoints at block boundaries
 * ("Hybrid transformers under load", section 3: reusing a shared prefix needs
 * a saved copy of the state where the prefix ends, since the live state goes
 * on to absorb the rest of the request; section 4.2: such snapshots are taken
 * at every cache-block boundary, 528 tokens there; section 6.1 measures their
 * cost).  Everything gdn_prefill_chunked computes and writes is computed and
 * written the same way, bit for bit; in addition, for each sequence s and
 * each p = ckpt_every, 2 ckpt_every, ... <= n_s, the state after the first p
 * tokens of s (counted within this call) is written to
 *   ckpt fp32 [n_ckpt][H_v][d_v][d_k],
 * numbered sequence by sequence in token order: sequence s's checkpoints start
 * at index sum over s' < s of floor(n_s' / ckpt_every).  A sequence whose
 * length is a multiple of ckpt_every ends on a checkpoint equal to its final
 * state.  The conv history at checkpoint p is not written: it is the input
 * rows x[cu_seqlens[s] + p - W + 1 .. cu_seqlens[s] + p - 1] (for p >= W-1;
 * earlier rows come from the sequence's initial history), which the caller
 * holds.  Entries past the last checkpoint are not touched.
 *   ckpt_every: any positive number of tokens (a block may end inside a chunk).
 *   ckpt: device, 16-byte aligned, ckpt_bytes >= floor(n_tokens / ckpt_every)
 *   * H_v * d_v * d_k * 4 (no partition of n_tokens has more checkpoints);
 *   NULL only when that bound is 0.
 * Errors as gdn_prefill_chunked, plus GDN_ERR_RANGE for ckpt_every and
 * ckpt_bytes.
 */
gdn_status gdn_prefill_chunked_ckpt(const gdn_geometry* g, float* state, float* conv_state,
                                    int32_t* conv_pos, const void* x, const void* a, const void* b,
                                    const float* conv_w, const int32_t* cu_seqlens,
                                    const int32_t* slot, const int32_t* has_init, int32_t n_seqs,
                                    int32_t n_tokens, int32_t chunk, void* workspace,
                                    size_t workspace_bytes, void* o, int32_t ckpt_every,
                                    float* ckpt, size_t ckpt_bytes, int32_t* dev_err,
                                    void* stream);

/*
 * Kernel timing, for measurement: the next gdn_prefill_chunked,
 * gdn_prefill_chunked_static or gdn_prefill_chunked_ckpt call made on this
 * host thread records `start` when its small plan kernel completes, which is
 * where its main kernel begins, and `stop` when its last main kernel
 * completes, through the kernel launches themselves (hipExtLaunchKernel), so
 * no event packet is put between the call's kernels and the caller's.  The
 * interval is the main kernel's run (the plan kernel, about 4 us, precedes
 * it).  `start` and `stop` are hipEvent_t handles the caller created
 * beforehand and still owns.  The
 * request is consumed by that next prefill call, whatever its outcome; both
 * null clears it.  A prefill under graph capture with a request pending fails
 * with GDN_ERR_LAUNCH and launches nothing: an event recorded under capture
 * times nothing, and a measurement that would read as zero must refuse
 * ("Chapter 6: engine startup and memory plan", section 6.10, on the
 * stage-timing guard).  Host only, thread-local, launches nothing.
 * Errors: GDN_ERR_NULL when exactly one of the two is null.
 */
gdn_status gdn_prefill_timing_events(void* start, void* stop);

/*
 * Speculative verify of k draft tokens per batch row ("Forge", 27 August:
 * the DeltaNet state walks the draft rows in order, with a snapshot of the
 * state after every row).  For draft j = 0..k-1 it computes the same per-token
 * math as gdn_decode_step, bit for bit, and writes
 *   snap [batch][k][H_v][d_v][d_k] fp32 = state after draft j,
 *   o    [batch][k][H_v][d_v]      dtype_out.
 * The committed state and conv_pos are NOT modified; the drafts' inputs are
 * written into ring rows p .. p+k-1 ahead of the committed history.
 *   x [batch][k][C], a, b [batch][k][H_v] (dtype_in).  1 <= k <= max_draft.
 */
gdn_status gdn_verify_k(const gdn_geometry* g, const float* state, float* conv_state,
                        const int32_t* conv_pos, const void* x, const void* a, const void* b,
                        const float* conv_w, const int32_t* slot, int32_t batch, int32_t k,
                        float* snap, void* o, int32_t* dev_err, void* stream);

/*
 * Commit accepted drafts after gdn_verify_k (same slot, batch, k and snap):
 * for each batch row with n = accepted[i] (device int32 [batch], 0..k):
 * if n >= 1 the slot's state becomes a bitwise copy of snap[i][n-1] and
 * conv_pos advances n tokens; n = 0 leaves the slot unchanged.
 * ("Forge", 27 August: with a snapshot after every draft row, rolling the
 * recurrent state back to the last accepted draft is a copy, not a replay.)
 * An accepted length out of range sets GDN_DEV_BAD_ACCEPTED and the row is
 * skipped.
 */
gdn_status gdn_rollback(const gdn_geometry* g, float* state, int32_t* conv_pos,
                        const float* snap, const int32_t* slot, const int32_t* accepted,
                        int32_t batch, int32_t k, int32_t* dev_err, void* stream);

/*
 * Verify with zero-copy commit ("Forge", entry of 27 August: a snapshot of
 * the state after every draft row makes rollback a copy; here the snapshot
 * is a whole pool slot, so the commit copies nothing).  Computes exactly what
 * gdn_verify_k computes, bit for bit, but snapshot j of row i goes to pool
 * slot s_j = snap_slot[i][j] (device int32 [batch][k]) as a complete slot:
 *   state[s_j]      = state after draft j (fp32, as snap[i][j] of gdn_verify_k),
 *   conv ring of s_j = the W-1 inputs before position p+j+1 (committed history
 *                      and drafts), at their ring rows,
 *   conv_pos[s_j]   = p+j+1 tokens,
 * where p is slot[i]'s position.  slot[i]'s state and position are not
 * modified; its ring receives the drafts' inputs as in gdn_verify_k.  Any
 * earlier contents of the snapshot slots are overwritten.
 * Every slot id in slot[] and snap_slot[] must be distinct (undefined results
 * otherwise); a snapshot slot id out of range sets GDN_DEV_BAD_SLOT and that
 * snapshot is skipped.  batch * (k+1) <= n_slots.  A caller that verifies the
 * last accepted token together with its drafts passes them as k+1 rows.
 * Rows may verify different numbers of drafts: k_row (device int32 [batch],
 * or NULL for k on every row) gives row i's count k_i in 1..k; x, a, b and o
 * keep their [batch][k] layout, and rows j >= k_i are neither read nor
 * written, nor are snap_slot[i][j] for j >= k_i.  A count out of range sets
 * GDN_DEV_BAD_K and the row is skipped.
 */
gdn_status gdn_verify_k_slots(const gdn_geometry* g, float* state, float* conv_state,
                              int32_t* conv_pos, const void* x, const void* a, const void* b,
                              const float* conv_w, const int32_t* slot, int32_t batch, int32_t k,
                              const int32_t* k_row, const int32_t* snap_slot, void* o,
                              int32_t* dev_err, void* stream);

/*
 * Commit after gdn_verify_k_slots (same slot, k_row, snap_slot, batch and k):
 * for each row with n = accepted[i] (device int32 [batch], 0..k_i),
 *   next_slot[i] = snap_slot[i][n-1] if n >= 1, else slot[i]   (device int32 [batch]).
 * The row's sequence continues in next_slot[i]; nothing is copied.  The
 * other slots of the row (slot[i] when n >= 1, and the snapshot slots not
 * chosen) hold nothing the sequence needs any more.  An accepted length out
 * of range sets GDN_DEV_BAD_ACCEPTED (a draft count out of range,
 * GDN_DEV_BAD_K) and keeps slot[i].  ("Forge", 27 August: the accepted
 * draft's snapshot becomes the state the sequence continues from.)
 */
gdn_status gdn_commit_slots(const gdn_geometry* g, const int32_t* slot, const int32_t* k_row,
                            const int32_t* snap_slot, const int32_t* accepted, int32_t batch, int32_t k,
                            int32_t* next_slot, int32_t* dev_err, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
