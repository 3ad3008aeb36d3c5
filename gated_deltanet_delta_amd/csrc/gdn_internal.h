// Internal interface between the C-ABI layer (gdn_api.cpp) and the kernel
// launchers (gdn_step.hip, gdn_prefill.hip).  Host code only.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Arguments of the per-token kernels (decode, verify, conv step, rollback).
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
  int32_t seg_lo, seg_hi;  // chunk-table range of one launch segment (set by the launcher)
  int32_t persistent;      // 1: one chain launch over whole sequences, waiting on per-chunk ready flags
  float* ckpt;             // state checkpoints [n][Hv][D][D], or null
  int32_t ckpt_every;      // tokens between checkpoints (a multiple of kChunk), 0: none
};

// Byte offsets and block sizes of the prefill workspace.
//   kq:   per (chunk, k-head) block of packed Q operand tiles (kq_bytes each)
//   head: per (chunk, v-head) block of packed -W, decayed K^T, P, U', the gate factors and V (head_bytes each)
//   ready: per (chunk, k-head) flag, set once the chunk kernel has published that block
struct PrefillLayout {
  size_t kq, head, chunk_tab, seq_tab, ready, total;
  size_t kq_bytes, head_bytes;
};
PrefillLayout prefill_layout(int Hk, int Hv, int D, bool bf16, int max_chunks, int n_seqs);
int prefill_max_chunks(int n_tokens, int n_seqs);
constexpr int kChunk = 64;

// Launchers: return 0 on success, else the hipError_t value.
int launch_decode(const StepArgs& a, bool bf16, void* stream);
int launch_verify(const StepArgs& a, bool bf16, void* stream);
int launch_conv_step(const StepArgs& a, bool bf16, void* stream);
int launch_rollback(const StepArgs& a, void* stream);
int launch_commit_slots(const StepArgs& a, void* stream);
int launch_prefill(const PrefillArgs& a, bool bf16, void* stream);

}  // namespace gdn
