// Internal interface between the C-ABI layer (gdn_api.cpp) and the kernel
// launchers (gdn_step.hip, gdn_prefill.hip).  Host code only.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Arguments of the per-token kernels (decode, verify, conv step, rollback).
// Work split of the decode and verify step: one workgroup per (batch row,
// v-head, block of state rows); a state row (d_k floats) is read by LPR lanes
// as one f32x4 each.  Shared by the kernels and by the host's launch checks.
template <int D, bool VERIFY>
struct StepShape {
  static constexpr int kWaveLanes = 64;
  static constexpr int LPR = D / 4;                   // lanes per state row (one f32x4 each)
  static constexpr int RPW = kWaveLanes / LPR;        // rows one wave covers per pass
  static constexpr int NP = D >= 64 ? 4 : (D >= 32 ? 2 : 1);  // passes per wave
  static constexpr int ROWS_WAVE = RPW * NP;
  static constexpr int NW_MAX = D / ROWS_WAVE;
  // waves per workgroup.  Decode: 8 (64 rows), which halves the workgroups
  // that add a share of the slot's position with one contended atomic;
  // verify (no position update, k drafts per workgroup): 4.
  static constexpr int NW = NW_MAX < (VERIFY ? 4 : 8) ? NW_MAX : (VERIFY ? 4 : 8);
  static constexpr int ROWS_WG = NW * ROWS_WAVE;
  static constexpr int WG_PER_HEAD = D / ROWS_WG;
  static constexpr int THREADS = NW * kWaveLanes;
};

// workgroups of one decode call on one slot (d_k = 16, 32, 64 or 128; 0 otherwise)
inline int decode_wgs_per_slot(int d_k, int n_v_heads) {
  switch (d_k) {
    case 16: return n_v_heads * StepShape<16, false>::WG_PER_HEAD;
    case 32: return n_v_heads * StepShape<32, false>::WG_PER_HEAD;
    case 64: return n_v_heads * StepShape<64, false>::WG_PER_HEAD;
    case 128: return n_v_heads * StepShape<128, false>::WG_PER_HEAD;
    default: return 0;
  }
}

struct StepArgs {
  float* state;          // decode: in/out; verify: in; rollback: out
  float* conv_state;
  int32_t* conv_pos;
  const void* x;
  const void* a;
  const void* b;
  const float* conv_w;
  const int32_t* slot;
  const int32_t* accepted;  // rollback only
  void* o;                  // o, or y for the conv step
  float* snap;              // verify: out; rollback: in
  const int32_t* snap_slot; // verify into pool slots: [batch][k] slots receiving the snapshots (else null)
  const int32_t* k_row;     // verify into pool slots, commit: drafts of each row (null: k for every row)
  int32_t* next_slot;       // slot commit: out
  int32_t* dev_err;
  int32_t batch, k;
  int32_t Hk, Hv, D, C, W, R, n_slots;
  uint32_t flags;
  float q_scale, l2_eps;
};

struct PrefillArgs {
  float* state;
  float* conv_state;
  int32_t* conv_pos;
  const void* x;
  const void* a;
  const void* b;
  const float* conv_w;
  const int32_t* cu_seqlens;
  const int32_t* slot;
  const int32_t* has_init;
  void* o;
  int32_t* dev_err;
  void* workspace;
  int32_t n_seqs, n_tokens, max_chunks;
  int32_t Hk, Hv, D, C, W, R, n_slots;
  uint32_t flags;
  float q_scale, l2_eps;
  float* ckpt;             // state checkpoints [n][Hv][D][D], or null
  int32_t ckpt_every;      // tokens between checkpoints, 0: none
  // set by the launcher for each launch of the fused kernel
  int32_t kh_lo, kh_hi;    // k-heads [kh_lo, kh_hi) of this launch
  int32_t seg;             // launch index (selects its counters)
  int32_t last_seg;        // 1 on the launch that writes the ring positions
};

// Byte offsets of the prefill workspace.  Its size does not depend on the
// number of tokens: chunks pass from producer to chain workgroups through a
// ring of ring_slots chunk slots.
//   ring:     [ring_slots][Hk] blocks of item_bytes (packed operands of one (chunk, k-head))
//   hdr:      total chunk count and the abort word
//   seq_tab:  per-sequence table (int32 x 8 each)
//   ready:    per (ring slot, k-head) publish flag = chunk + 1, one 128-byte line each
//   consumed: per v-head, chunks staged by its chain workgroup, one line each
//   ctr:      per launch: role and item tickets per XCD, the exit word
struct PrefillLayout {
  size_t ring, hdr, seq_tab, ready, consumed, ctr, total;
  size_t item_bytes;
  int32_t ring_slots;
};
PrefillLayout prefill_layout(int Hk, int Hv, int D, bool bf16, int n_tokens, int n_seqs);
int prefill_max_chunks(int n_tokens, int n_seqs);
int prefill_launches(int Hk, int Hv, int D, bool bf16);
constexpr int kChunk = 64;

// Launchers: return 0 on success, else the hipError_t value.
int launch_decode(const StepArgs& a, bool bf16, void* stream);
int launch_verify(const StepArgs& a, bool bf16, void* stream);
int launch_conv_step(const StepArgs& a, bool bf16, void* stream);
int launch_rollback(const StepArgs& a, void* stream);
int launch_commit_slots(const StepArgs& a, void* stream);
// Debug builds: one small kernel reporting GDN_DEV_DUP_SLOT to *dev_err when
// two of a call's slot ids are equal: a[0..na), then, for rows i < nb, the
// ids b[i kb + j] for j < kb, or j < k_row[i] when k_row is given (rows whose
// count is out of range are left out).  Nothing is launched without dev_err.
int launch_check_distinct(const int32_t* a, int na, const int32_t* b, int nb, int kb, const int32_t* k_row,
                          int32_t* dev_err, void* stream);
// ev_start / ev_stop (hipEvent_t, optional): recorded by the call's kernel
// launches themselves, when the plan kernel ends (the main kernel begins) and
// when the last main kernel ends.
int launch_prefill(const PrefillArgs& a, bool bf16, void* stream, void* ev_start = nullptr, void* ev_stop = nullptr);
// Device address of the library's static prefill workspace on the GPU of
// `stream` (GDN_PREFILL_STATIC_WORKSPACE_BYTES); a HIP error code, 0 on success.
int prefill_static_workspace(void* stream, void** ptr);

}  // namespace gdn
