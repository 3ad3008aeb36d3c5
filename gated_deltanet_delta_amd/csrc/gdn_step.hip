// Per-token GDN kernels for gfx950: fused decode step, k-draft verify with
// per-draft snapshots, the standalone conv-ring step, and rollback.
//
// The rule (Gated DeltaNet, arXiv:2412.06464; described in words in "Hybrid
// transformers under load", section 3):
//   S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T,   o_t = S_t q_t.
// Per state row i (length d_k) this is, with s_k = S_i.k and s_q = S_i.q of the
// OLD row,
//   u_i = beta (v_i - alpha s_k),  S_i <- alpha S_i + u_i k,
//   o_i = alpha s_q + u_i (k.q)          (= (S_t q)_i exactly in real arithmetic),
// so every fp32 state row is read once and written once: decode is bound by
// HBM bandwidth, and the kernel streams rows through registers with 16-byte
// coalesced loads and non-temporal stores.
//
// Work split: one workgroup per (batch row, v-head, block of state rows).
// Every wave computes the conv front end of the q and k channels of its
// k-head itself (each lane the 4 columns it multiplies), so no LDS and no
// barrier sits between the state loads and the row updates.  Decode and
// verify are the same template, so verify's per-draft math is bit-identical
// to decode's (rollback to a snapshot equals a decode replay, bit for bit).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Input of the conv window at relative token `rel` (rel >= 0: token rel of
// this batch row; rel < 0: ring row of position pos + rel).
template <bool BF16>
__device__ __forceinline__ float window_in1(const float* ring, uint32_t pos, int R,
                                            const void* xb, int C, int rel, int c) {
  if (rel >= 0) return load_in<BF16>(xb, static_cast<size_t>(rel) * C + c);
  return ring[static_cast<size_t>(ring_row(pos + static_cast<uint32_t>(rel), R)) * C + c];
}

// Causal depthwise conv (taps oldest first, tap W-1 on token j) + SiLU of
// channel c.  W is a compile-time constant so that every tap's loads are
// issued together; W == 0 passes the input through.
template <bool BF16, int W>
__device__ __forceinline__ float conv1(const float* ring, uint32_t pos, int R, const void* xb,
                                       int C, const float* w, int j, int c) {
  if constexpr (W == 0) {
    return load_in<BF16>(xb, static_cast<size_t>(j) * C + c);
  } else {
    float in[W], wt[W];
#pragma unroll
    for (int t = 0; t < W; ++t) in[t] = window_in1<BF16>(ring, pos, R, xb, C, j - (W - 1) + t, c);
    if constexpr (W == 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(w + c * 4);
      wt[0] = w4.x; wt[1] = w4.y; wt[2] = w4.z; wt[3] = w4.w;
    } else {
#pragma unroll
      for (int t = 0; t < W; ++t) wt[t] = w[c * W + t];
    }
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < W; ++t) acc = fmaf(wt[t], in[t], acc);
    return silu_f(acc);
  }
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
  float s = a.x * b.x;
  s = fmaf(a.y, b.y, s);
  s = fmaf(a.z, b.z, s);
  return fmaf(a.w, b.w, s);
}

__device__ __forceinline__ float dot4v(f32x4_t a, float4 b) {
  float s = a.x * b.x;
  s = fmaf(a.y, b.y, s);
  s = fmaf(a.z, b.z, s);
  return fmaf(a.w, b.w, s);
}

// Decode (VERIFY = false: k = 1, state updated in place, position advanced)
// and verify (VERIFY = true: k drafts, snapshot after each, state untouched).
//
// The conv front end is shared by the workgroup: thread t < 2 d_k computes
// q / k channel t of the k-head, thread t < ROWS_WG the v channel of row t of
// the workgroup's block, each with its own sliding conv window; results go
// through a small LDS table (an LDS-only barrier, which leaves the state
// loads in flight).  Then every lane group updates its state rows as before.
//
// Memory order of a call: the slot id and everything that does not depend on
// it (this token's inputs, conv weights, gates) are requested first; then the
// ring position; then the state rows (pinned ahead of all arithmetic by a
// scheduling barrier, so their HBM latency overlaps the rest), with
// non-temporal loads (each state row is read once per call); then the W-1
// ring rows of the conv window.  (Reading all ring rows before the state, to
// skip the wait on the position, measured slower: it puts the ring's bytes
// ahead of the state's in the memory queues.)
template <int D, bool BF16, bool VERIFY, int W>
__global__ __launch_bounds__((StepShape<D, VERIFY>::THREADS)) void step_kernel(StepArgs A) {
  using Sh = StepShape<D, VERIFY>;
  constexpr int LPR = Sh::LPR;
  constexpr int NP = Sh::NP;
  constexpr int NG = D < kWave ? D : kWave;            // lanes per partial sum of squares
  static_assert(Sh::THREADS >= 2 * D && Sh::THREADS >= Sh::ROWS_WG, "one channel per thread");
  __shared__ float fe[2][2 * D + Sh::ROWS_WG];         // q | k | v of a token (two tokens in flight)
  __shared__ float ssq[2][2 * D / NG];                 // partial sums of squares of q and k
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int hb = blockIdx.x % Sh::WG_PER_HEAD;
  const int h = blockIdx.x / Sh::WG_PER_HEAD;
  const int b = blockIdx.y;
  const int slot_in = A.slot[b];                       // requested first (scalar load)
  const int G = A.Hv / A.Hk;
  const int kh = h / G;
  const int c4 = (lane % LPR) * 4;                     // first state column of this lane
  const int rloc0 = wave * Sh::ROWS_WAVE + lane / LPR; // this lane's first row within the block
  const int row0 = hb * Sh::ROWS_WG + rloc0;
  const int R = A.R, C = A.C;
  const int kdr = VERIFY ? A.k : 1;
  const char* xb = static_cast<const char*>(A.x) + static_cast<size_t>(b) * kdr * C * (BF16 ? 2 : 4);
  const size_t xrow = static_cast<size_t>(C) * (BF16 ? 2 : 4);
  // the channel this thread runs the conv of: q / k of the k-head, or v of a row
  const bool fe_qk = tid < 2 * D;
  const bool fe_v = tid < Sh::ROWS_WG;
  const int ch_qk = tid < D ? kh * D + tid : A.Hk * D + kh * D + (tid - D);
  const int ch_v = 2 * A.Hk * D + h * D + hb * Sh::ROWS_WG + tid;
  const int chq = fe_qk ? ch_qk : 0, chv = fe_v ? ch_v : 0;  // clamped: every load stays in the row

  // ---- slot-independent inputs: token 0, conv weights, gates of token 0 ----
  float xq = load_in<BF16>(xb, chq), xv = load_in<BF16>(xb, chv);
  float4 wq = make_float4(0.f, 0.f, 0.f, 0.f), wv = wq;
  if constexpr (W == 4) {
    wq = *reinterpret_cast<const float4*>(A.conv_w + chq * 4);
    wv = *reinterpret_cast<const float4*>(A.conv_w + chv * 4);
  }
  size_t gi = static_cast<size_t>(b) * kdr * A.Hv + h;
  float ga = load_in<BF16>(A.a, gi), gb = load_in<BF16>(A.b, gi);

  // A bad slot id is reported and its row skipped; the loads below then read
  // slot 0 (harmless) so that no branch sits between the loads above and
  // their use (a branch would let the compiler sink them behind the slot).
  const bool slot_ok = slot_in >= 0 && slot_in < A.n_slots;
  if (!slot_ok && tid == 0 && blockIdx.x == 0) report_error(A.dev_err, GDN_DEV_BAD_SLOT);
  const int slot = slot_ok ? slot_in : 0;

  // ---- the ring position, then the state rows (the position is requested
  // first: loads complete in order, so the ring rows below wait for it alone) ----
  const uint32_t pos = W > 0 ? (static_cast<uint32_t>(A.conv_pos[slot * kPosStride]) >> kPosShift) : 0u;
  __builtin_amdgcn_sched_barrier(0);
  const float* Sg = A.state + (static_cast<size_t>(slot) * A.Hv + h) * D * D;
  f32x4_t S[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    S[p] = load_nt4(Sg + static_cast<size_t>(row0 + p * Sh::RPW) * D + c4);
  __builtin_amdgcn_sched_barrier(0);

  // ---- conv window history of this thread's channels: ring rows pos-3 .. pos-1 ----
  float hq[3] = {0.f, 0.f, 0.f}, hv[3] = {0.f, 0.f, 0.f};
  if constexpr (W == 4) {
    const float* ring = A.conv_state + static_cast<size_t>(slot) * R * C;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const float* rr = ring + static_cast<size_t>(ring_row(pos + static_cast<uint32_t>(t - 3), R)) * C;
      hq[t] = rr[chq];
      hv[t] = rr[chv];
    }
  }
  const bool qk_writer = fe_qk && (h % G == 0) && hb == 0 && slot_ok;
  const bool v_writer = fe_v && slot_ok;
  const bool o_writer = (lane % LPR) == 0 && slot_ok;
  // Verify into pool slots: snapshot j becomes a whole slot (state, conv
  // history, position) of its own, so a commit only has to pick a slot id.
  const bool to_slots = VERIFY && A.snap_slot != nullptr;
  // drafts of this row: k, or the row's own count (rows j >= kn of x, a, b
  // are not read, and their outputs and snapshots are not written)
  int kn = kdr;
  if (VERIFY && A.k_row != nullptr) {
    const int kr = A.k_row[b];
    if (kr < 1 || kr > kdr) {
      if (tid == 0 && blockIdx.x == 0) report_error(A.dev_err, GDN_DEV_BAD_K);
      kn = 0;
    } else {
      kn = kr;
    }
  }

  for (int j = 0; j < kn; ++j) {
    int ss = 0;
    bool ss_ok = false;
    if (to_slots) {
      const int ss_in = A.snap_slot[static_cast<size_t>(b) * kdr + j];
      ss_ok = slot_ok && ss_in >= 0 && ss_in < A.n_slots;
      if (!ss_ok && slot_ok && tid == 0 && blockIdx.x == 0) report_error(A.dev_err, GDN_DEV_BAD_SLOT);
      ss = ss_ok ? ss_in : 0;
    }
    // next draft's inputs (verify), requested before this draft's arithmetic
    float nxq = xq, nxv = xv, na = ga, nb = gb;
    if (VERIFY && j + 1 < kn) {
      nxq = load_in<BF16>(xb + (j + 1) * xrow, chq);
      nxv = load_in<BF16>(xb + (j + 1) * xrow, chv);
      na = load_in<BF16>(A.a, gi + A.Hv);
      nb = load_in<BF16>(A.b, gi + A.Hv);
    }
    // ---- front end, one channel per thread: conv + SiLU, sums of squares ----
    float* f = fe[j & 1];
    float yq, yv;
    if constexpr (W == 4) {
      yq = silu_fast(fmaf(wq.w, xq, fmaf(wq.z, hq[2], fmaf(wq.y, hq[1], wq.x * hq[0]))));
      yv = silu_fast(fmaf(wv.w, xv, fmaf(wv.z, hv[2], fmaf(wv.y, hv[1], wv.x * hv[0]))));
      hq[0] = hq[1]; hq[1] = hq[2]; hq[2] = xq;
      hv[0] = hv[1]; hv[1] = hv[2]; hv[2] = xv;
      if (to_slots && ss_ok) {
        // the snapshot slot's history: tokens pos+j-2 .. pos+j, at their ring rows
        float* sring = A.conv_state + static_cast<size_t>(ss) * R * C;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          float* rr = sring + static_cast<size_t>(ring_row(pos + static_cast<uint32_t>(j + t) - 2u, R)) * C;
          if (qk_writer) rr[chq] = hq[t];
          if (v_writer) rr[chv] = hv[t];
        }
        if (h == 0 && hb == 0 && tid == 0)
          A.conv_pos[ss * kPosStride] = static_cast<int32_t>((pos + static_cast<uint32_t>(j + 1)) << kPosShift);
      }
    } else {
      yq = xq;
      yv = xv;
    }
    float sq = group_sum<NG < 32 ? NG : 32>(yq * yq);
    if constexpr (NG == 64)  // the two 32-lane halves, added in a fixed order
      sq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sq), 0)) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sq), 32));
    if (fe_qk) {
      f[tid] = yq;
      if (tid % NG == 0) ssq[j & 1][tid / NG] = sq;
    }
    if (fe_v) f[2 * D + tid] = yv;
    // ---- append this token's raw input to the ring (rows nobody reads now) ----
    if constexpr (W > 0) {
      float* rrow = A.conv_state + (static_cast<size_t>(slot) * R + ring_row(pos + j, R)) * C;
      if (qk_writer) rrow[chq] = xq;
      if (v_writer) rrow[chv] = xv;
    }
    lds_barrier();
    if (!VERIFY && W > 0 && j == 0 && slot_ok && tid == 0) {
      // Advance the position by this workgroup's share of one token.  Every
      // wave of the workgroup has its position load completed (it picked its
      // window rows before the barrier above); the shares of the slot's
      // workgroups sum to exactly 1 << kPosShift and no partial sum reaches it,
      // so every reader of this call sees the same position.
      const uint32_t nwg = gridDim.x;
      const uint32_t one = 1u << kPosShift;
      const uint32_t share = one / nwg + (blockIdx.x < one % nwg ? 1u : 0u);
      atomicAdd(reinterpret_cast<unsigned int*>(A.conv_pos + slot * kPosStride), share);
    }
    // ---- L2 norm of q and k, gates ----
    float sqq = 0.f, skk = 0.f;
#pragma unroll
    for (int i = 0; i < D / NG; ++i) {
      sqq += ssq[j & 1][i];
      skk += ssq[j & 1][D / NG + i];
    }
    float qs = A.q_scale, ks = 1.0f;
    if (A.flags & GDN_FLAG_L2NORM_QK) {
      qs = qs * __builtin_amdgcn_rsqf(sqq + A.l2_eps);
      ks = __builtin_amdgcn_rsqf(skk + A.l2_eps);
    }
    const float4 qr = *reinterpret_cast<const float4*>(f + c4);
    const float4 kr = *reinterpret_cast<const float4*>(f + D + c4);
    const float4 q = make_float4(qr.x * qs, qr.y * qs, qr.z * qs, qr.w * qs);
    const float4 k = make_float4(kr.x * ks, kr.y * ks, kr.z * ks, kr.w * ks);
    const float kq = group_sum<LPR>(dot4(k, q));
    // alpha = exp(-softplus(a)) = 1 / (1 + e^a) = sigmoid(-a); beta = sigmoid(b)
    const float alpha = sigmoid_fast(-ga);
    const float beta = sigmoid_fast(gb);

    // ---- rank-1 delta update and output, one state row per lane group ----
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = row0 + p * Sh::RPW;
      const float v = f[2 * D + rloc0 + p * Sh::RPW];
      const float sk = group_sum<LPR>(dot4v(S[p], k));
      const float sqv = group_sum<LPR>(dot4v(S[p], q));
      const float u = beta * (v - alpha * sk);
      const float ov = fmaf(alpha, sqv, u * kq);
      f32x4_t sn;
      sn.x = fmaf(u, k.x, alpha * S[p].x);
      sn.y = fmaf(u, k.y, alpha * S[p].y);
      sn.z = fmaf(u, k.z, alpha * S[p].z);
      sn.w = fmaf(u, k.w, alpha * S[p].w);
      S[p] = sn;
      if (!VERIFY && slot_ok)
        store_nt4(A.state + (static_cast<size_t>(slot) * A.Hv + h) * D * D + static_cast<size_t>(row) * D + c4, sn);
      if (VERIFY && slot_ok && !to_slots) {
        float* dst = A.snap + ((((static_cast<size_t>(b) * kdr + j) * A.Hv + h) * D + row) * D + c4);
        store_nt4(dst, sn);
      }
      if (to_slots && ss_ok)
        store_nt4(A.state + (static_cast<size_t>(ss) * A.Hv + h) * D * D + static_cast<size_t>(row) * D + c4, sn);
      if (o_writer) store_out<BF16>(A.o, (gi * D) + row, ov);
    }
    xq = nxq;
    xv = nxv;
    ga = na;
    gb = nb;
    gi += A.Hv;
  }

}

// Standalone conv-ring step over all C channels: y = SiLU(conv), append x.
template <bool BF16, int W>
__global__ __launch_bounds__(256) void conv_step_kernel(StepArgs A) {
  const int b = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int slot = A.slot[b];
  if (slot < 0 || slot >= A.n_slots) {
    if (threadIdx.x == 0 && blockIdx.x == 0) report_error(A.dev_err, GDN_DEV_BAD_SLOT);
    return;
  }
  const int C = A.C, R = A.R;
  const float* ring = A.conv_state + static_cast<size_t>(slot) * R * C;
  const uint32_t pos = static_cast<uint32_t>(A.conv_pos[slot * kPosStride]) >> kPosShift;
  const void* xb = static_cast<const char*>(A.x) + static_cast<size_t>(b) * C * (BF16 ? 2 : 4);
  if (c < C) {
    const float y = conv1<BF16, W>(ring, pos, R, xb, C, A.conv_w, 0, c);
    store_out<BF16>(A.o, static_cast<size_t>(b) * C + c, y);
    A.conv_state[(static_cast<size_t>(slot) * R + ring_row(pos, R)) * C + c] = load_in<BF16>(xb, c);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t nwg = gridDim.x;
    const uint32_t one = 1u << kPosShift;
    const uint32_t share = one / nwg + (blockIdx.x < one % nwg ? 1u : 0u);
    atomicAdd(reinterpret_cast<unsigned int*>(A.conv_pos + slot * kPosStride), share);
  }
}

// Commit: state[slot] <- snap[b][n-1] (bitwise), position += n tokens.
constexpr int kRollbackVecsPerThread = 4;
__global__ __launch_bounds__(256) void rollback_kernel(StepArgs A) {
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int slot = A.slot[b];
  const int n = A.accepted[b];
  if (slot < 0 || slot >= A.n_slots) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && h == 0) report_error(A.dev_err, GDN_DEV_BAD_SLOT);
    return;
  }
  if (n < 0 || n > A.k) {
    if (threadIdx.x == 0 && blockIdx.x == 0 && h == 0) report_error(A.dev_err, GDN_DEV_BAD_ACCEPTED);
    return;
  }
  if (n == 0) return;
  const size_t head = static_cast<size_t>(A.D) * A.D;
  const float* src = A.snap + ((static_cast<size_t>(b) * A.k + (n - 1)) * A.Hv + h) * head;
  float* dst = A.state + (static_cast<size_t>(slot) * A.Hv + h) * head;
  const size_t nvec = head / 4;
#pragma unroll
  for (int i = 0; i < kRollbackVecsPerThread; ++i) {
    const size_t e = (static_cast<size_t>(blockIdx.x) * kRollbackVecsPerThread + i) * 256 + threadIdx.x;
    if (e < nvec) store_nt4(dst + e * 4, load4(src + e * 4));
  }
  if (A.W > 0 && h == 0 && blockIdx.x == 0 && threadIdx.x == 0)
    A.conv_pos[slot * kPosStride] = static_cast<int32_t>(static_cast<uint32_t>(A.conv_pos[slot * kPosStride]) +
                                            (static_cast<uint32_t>(n) << kPosShift));
}

// Commit after a verify into pool slots: the row's sequence continues in the
// slot that holds the state after its last accepted draft (its own slot when
// none was accepted).  Nothing is copied.
__global__ __launch_bounds__(256) void commit_slots_kernel(StepArgs A) {
  for (int b = blockIdx.x * 256 + threadIdx.x; b < A.batch; b += gridDim.x * 256) {
    const int n = A.accepted[b];
    const int kr = A.k_row != nullptr ? A.k_row[b] : A.k;
    int out = A.slot[b];
    if (kr < 1 || kr > A.k) report_error(A.dev_err, GDN_DEV_BAD_K);
    else if (n < 0 || n > kr) report_error(A.dev_err, GDN_DEV_BAD_ACCEPTED);
    else if (n > 0) out = A.snap_slot[static_cast<size_t>(b) * A.k + (n - 1)];
    A.next_slot[b] = out;
  }
}

// Debug builds: two equal slot ids in one call (every id against every earlier one).
__global__ __launch_bounds__(256) void distinct_slots_kernel(const int32_t* a, int na, const int32_t* b, int nb,
                                                             int kb, const int32_t* k_row, int32_t* dev_err) {
  const int n = na + nb * kb;
  auto id = [&](int e, bool& used) {
    if (e < na) {
      used = true;
      return a[e];
    }
    const int i = (e - na) / kb, j = (e - na) % kb;
    const int kr = k_row != nullptr ? k_row[i] : kb;
    used = kr >= 1 && kr <= kb && j < kr;
    return used ? b[static_cast<size_t>(i) * kb + j] : 0;
  };
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    bool ue = false;
    const int ve = id(e, ue);
    if (!ue) continue;
    for (int f = 0; f < e; ++f) {
      bool uf = false;
      const int vf = id(f, uf);
      if (uf && vf == ve) {
        report_error(dev_err, GDN_DEV_DUP_SLOT);
        break;
      }
    }
  }
}

int launch_check_distinct(const int32_t* a, int na, const int32_t* b, int nb, int kb, const int32_t* k_row,
                          int32_t* dev_err, void* stream) {
  if (dev_err == nullptr || na + (b != nullptr ? nb * kb : 0) < 2) return 0;
  if (b == nullptr) nb = 0;
  hipLaunchKernelGGL(distinct_slots_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream), a, na, b, nb,
                     kb > 0 ? kb : 1, k_row, dev_err);
  return static_cast<int>(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool VERIFY>
static int launch_step_t(const StepArgs& a, hipStream_t s) {
  using Sh = StepShape<D, VERIFY>;
  dim3 grid(a.Hv * Sh::WG_PER_HEAD, a.batch);
  if (a.W == 4) hipLaunchKernelGGL((step_kernel<D, BF16, VERIFY, 4>), grid, dim3(Sh::THREADS), 0, s, a);
  else if (a.W == 0) hipLaunchKernelGGL((step_kernel<D, BF16, VERIFY, 0>), grid, dim3(Sh::THREADS), 0, s, a);
  else return static_cast<int>(hipErrorInvalidValue);
  return static_cast<int>(hipGetLastError());
}

template <bool VERIFY>
static int launch_step(const StepArgs& a, bool bf16, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.D) {
    case 16: return bf16 ? launch_step_t<16, true, VERIFY>(a, s) : launch_step_t<16, false, VERIFY>(a, s);
    case 32: return bf16 ? launch_step_t<32, true, VERIFY>(a, s) : launch_step_t<32, false, VERIFY>(a, s);
    case 64: return bf16 ? launch_step_t<64, true, VERIFY>(a, s) : launch_step_t<64, false, VERIFY>(a, s);
    case 128: return bf16 ? launch_step_t<128, true, VERIFY>(a, s) : launch_step_t<128, false, VERIFY>(a, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

int launch_decode(const StepArgs& a, bool bf16, void* stream) { return launch_step<false>(a, bf16, stream); }
int launch_verify(const StepArgs& a, bool bf16, void* stream) { return launch_step<true>(a, bf16, stream); }

int launch_conv_step(const StepArgs& a, bool bf16, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((a.C + 255) / 256, a.batch);
  if (a.W != 4) return static_cast<int>(hipErrorInvalidValue);
  if (bf16) hipLaunchKernelGGL((conv_step_kernel<true, 4>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((conv_step_kernel<false, 4>), grid, dim3(256), 0, s, a);
  return static_cast<int>(hipGetLastError());
}

int launch_commit_slots(const StepArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int wgs = (a.batch + 255) / 256;
  hipLaunchKernelGGL(commit_slots_kernel, dim3(wgs < 64 ? wgs : 64), dim3(256), 0, s, a);
  return static_cast<int>(hipGetLastError());
}

int launch_rollback(const StepArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t nvec = static_cast<size_t>(a.D) * a.D / 4;
  const int per_wg = 256 * kRollbackVecsPerThread;
  dim3 grid(static_cast<unsigned>((nvec + per_wg - 1) / per_wg), a.Hv, a.batch);
  hipLaunchKernelGGL(rollback_kernel, grid, dim3(256), 0, s, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdn
