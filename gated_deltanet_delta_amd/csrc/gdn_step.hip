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

template <int D>
struct StepShape {
  static constexpr int LPR = D / 4;              // lanes per state row (one f32x4 each)
  static constexpr int RPW = kWave / LPR;        // rows one wave covers per pass
  static constexpr int NP = D >= 64 ? 4 : (D >= 32 ? 2 : 1);  // passes per wave
  static constexpr int ROWS_WAVE = RPW * NP;
  static constexpr int NW_MAX = D / ROWS_WAVE;
  static constexpr int NW = NW_MAX < 4 ? NW_MAX : 4;          // waves per workgroup
  static constexpr int ROWS_WG = NW * ROWS_WAVE;
  static constexpr int WG_PER_HEAD = D / ROWS_WG;
  static constexpr int THREADS = NW * kWave;
};

// Input of the conv window at relative token `rel` (rel >= 0: draft/current
// token rel of this batch row; rel < 0: ring row of position pos + rel).
template <bool BF16>
__device__ __forceinline__ float4 window_in4(const float* ring, uint32_t pos, int R,
                                             const void* xb, int C, int rel, int c) {
  if (rel >= 0) return load_in4<BF16>(xb, static_cast<size_t>(rel) * C + c);
  return *reinterpret_cast<const float4*>(
      ring + static_cast<size_t>(ring_row(pos + static_cast<uint32_t>(rel), R)) * C + c);
}

template <bool BF16>
__device__ __forceinline__ float window_in1(const float* ring, uint32_t pos, int R,
                                            const void* xb, int C, int rel, int c) {
  if (rel >= 0) return load_in<BF16>(xb, static_cast<size_t>(rel) * C + c);
  return ring[static_cast<size_t>(ring_row(pos + static_cast<uint32_t>(rel), R)) * C + c];
}

// Causal depthwise conv (taps oldest first, tap W-1 on token j) + SiLU for
// channels c..c+3.  W is a compile-time constant so that every tap's loads are
// issued together; W == 0 passes the input through.
template <bool BF16, int W>
__device__ __forceinline__ float4 conv4(const float* ring, uint32_t pos, int R, const void* xb,
                                        int C, const float* w, int j, int c) {
  if constexpr (W == 0) {
    return load_in4<BF16>(xb, static_cast<size_t>(j) * C + c);
  } else {
    float4 in[W];
    float wt[4][W];
#pragma unroll
    for (int t = 0; t < W; ++t) in[t] = window_in4<BF16>(ring, pos, R, xb, C, j - (W - 1) + t, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (W == 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(w + (c + i) * 4);
        wt[i][0] = w4.x; wt[i][1] = w4.y; wt[i][2] = w4.z; wt[i][3] = w4.w;
      } else {
#pragma unroll
        for (int t = 0; t < W; ++t) wt[i][t] = w[(c + i) * W + t];
      }
    }
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < W; ++t) {
      acc.x = fmaf(wt[0][t], in[t].x, acc.x);
      acc.y = fmaf(wt[1][t], in[t].y, acc.y);
      acc.z = fmaf(wt[2][t], in[t].z, acc.z);
      acc.w = fmaf(wt[3][t], in[t].w, acc.w);
    }
    return make_float4(silu_f(acc.x), silu_f(acc.y), silu_f(acc.z), silu_f(acc.w));
  }
}

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
template <int D, bool BF16, bool VERIFY, int W>
__global__ __launch_bounds__(StepShape<D>::THREADS) void step_kernel(StepArgs A) {
  using Sh = StepShape<D>;
  constexpr int LPR = Sh::LPR;
  constexpr int NP = Sh::NP;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int hb = blockIdx.x % Sh::WG_PER_HEAD;
  const int h = blockIdx.x / Sh::WG_PER_HEAD;
  const int b = blockIdx.y;
  const int G = A.Hv / A.Hk;
  const int kh = h / G;
  const int c4 = (lane % LPR) * 4;                  // first state column of this lane
  const int row0 = hb * Sh::ROWS_WG + wave * Sh::ROWS_WAVE + lane / LPR;

  const int slot = A.slot[b];
  if (slot < 0 || slot >= A.n_slots) {
    if (threadIdx.x == 0 && blockIdx.x == 0) report_error(A.dev_err, GDN_DEV_BAD_SLOT);
    return;
  }

  // Issue the state loads first; nothing below waits on them until the row loop.
  const float* Sg = A.state + (static_cast<size_t>(slot) * A.Hv + h) * D * D;
  f32x4_t S[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    S[p] = load4(Sg + static_cast<size_t>(row0 + p * Sh::RPW) * D + c4);

  const int R = A.R, C = A.C;
  const float* ring = W > 0 ? A.conv_state + static_cast<size_t>(slot) * R * C : nullptr;
  const uint32_t pos = W > 0 ? (static_cast<uint32_t>(A.conv_pos[slot]) >> kPosShift) : 0u;
  const int kdr = VERIFY ? A.k : 1;
  const void* xb = static_cast<const char*>(A.x) +
                   static_cast<size_t>(b) * kdr * C * (BF16 ? 2 : 4);
  const int cq = kh * D + c4;                         // q channels of this lane
  const int ck = A.Hk * D + kh * D + c4;              // k channels of this lane
  const int cv0 = 2 * A.Hk * D + h * D;               // v channels of this head
  const bool qk_writer = (h % G == 0) && hb == 0 && wave == 0 && lane < LPR;
  const bool v_writer = (lane % LPR) == 0;

  for (int j = 0; j < kdr; ++j) {
    // ---- front end: conv + SiLU, L2 norm of q and k, gates ----
    float4 q = conv4<BF16, W>(ring, pos, R, xb, C, A.conv_w, j, cq);
    float4 k = conv4<BF16, W>(ring, pos, R, xb, C, A.conv_w, j, ck);
    float qs = A.q_scale, ks = 1.0f;
    if (A.flags & GDN_FLAG_L2NORM_QK) {
      const float sqq = group_sum<LPR>(dot4(q, q));
      const float skk = group_sum<LPR>(dot4(k, k));
      qs = qs * (1.0f / sqrtf(sqq + A.l2_eps));
      ks = 1.0f / sqrtf(skk + A.l2_eps);
    }
    q = make_float4(q.x * qs, q.y * qs, q.z * qs, q.w * qs);
    k = make_float4(k.x * ks, k.y * ks, k.z * ks, k.w * ks);
    const float kq = group_sum<LPR>(dot4(k, q));
    float v[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
      v[p] = conv1<BF16, W>(ring, pos, R, xb, C, A.conv_w, j, cv0 + row0 + p * Sh::RPW);
    const size_t gi = (static_cast<size_t>(b) * kdr + j) * A.Hv + h;
    const float alpha = expf(-softplus_f(load_in<BF16>(A.a, gi)));
    const float beta = sigmoid_f(load_in<BF16>(A.b, gi));

    // ---- append this token's raw input to the ring (rows nobody reads now) ----
    if constexpr (W > 0) {
      float* rrow = A.conv_state + (static_cast<size_t>(slot) * R + ring_row(pos + j, R)) * C;
      if (qk_writer) {
        *reinterpret_cast<float4*>(rrow + cq) = load_in4<BF16>(xb, static_cast<size_t>(j) * C + cq);
        *reinterpret_cast<float4*>(rrow + ck) = load_in4<BF16>(xb, static_cast<size_t>(j) * C + ck);
      }
      if (v_writer) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int c = cv0 + row0 + p * Sh::RPW;
          rrow[c] = load_in<BF16>(xb, static_cast<size_t>(j) * C + c);
        }
      }
    }

    // ---- rank-1 delta update and output, one state row per lane group ----
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = row0 + p * Sh::RPW;
      const float sk = group_sum<LPR>(dot4v(S[p], k));
      const float sq = group_sum<LPR>(dot4v(S[p], q));
      const float u = beta * (v[p] - alpha * sk);
      const float ov = fmaf(alpha, sq, u * kq);
      f32x4_t sn;
      sn.x = fmaf(u, k.x, alpha * S[p].x);
      sn.y = fmaf(u, k.y, alpha * S[p].y);
      sn.z = fmaf(u, k.z, alpha * S[p].z);
      sn.w = fmaf(u, k.w, alpha * S[p].w);
      S[p] = sn;
      if (VERIFY) {
        float* dst = A.snap + ((((static_cast<size_t>(b) * kdr + j) * A.Hv + h) * D + row) * D + c4);
        store_nt4(dst, sn);
      }
      if (v_writer) store_out<BF16>(A.o, (gi * D) + row, ov);
    }
  }

  if (!VERIFY) {
    float* Sw = A.state + (static_cast<size_t>(slot) * A.Hv + h) * D * D;
#pragma unroll
    for (int p = 0; p < NP; ++p)
      store_nt4(Sw + static_cast<size_t>(row0 + p * Sh::RPW) * D + c4, S[p]);
    if constexpr (W > 0) {
      // Advance the position by this workgroup's share of one token; the
      // shares of the slot's workgroups sum to exactly 1 << kPosShift, and
      // no partial sum reaches it, so every reader of this call sees pos.
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t nwg = gridDim.x;
        const uint32_t one = 1u << kPosShift;
        const uint32_t share = one / nwg + (blockIdx.x < one % nwg ? 1u : 0u);
        atomicAdd(reinterpret_cast<unsigned int*>(A.conv_pos + slot), share);
      }
    }
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
  const uint32_t pos = static_cast<uint32_t>(A.conv_pos[slot]) >> kPosShift;
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
    atomicAdd(reinterpret_cast<unsigned int*>(A.conv_pos + slot), share);
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
    A.conv_pos[slot] = static_cast<int32_t>(static_cast<uint32_t>(A.conv_pos[slot]) +
                                            (static_cast<uint32_t>(n) << kPosShift));
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool VERIFY>
static int launch_step_t(const StepArgs& a, hipStream_t s) {
  using Sh = StepShape<D>;
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

int launch_rollback(const StepArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t nvec = static_cast<size_t>(a.D) * a.D / 4;
  const int per_wg = 256 * kRollbackVecsPerThread;
  dim3 grid(static_cast<unsigned>((nvec + per_wg - 1) / per_wg), a.Hv, a.batch);
  hipLaunchKernelGGL(rollback_kernel, grid, dim3(256), 0, s, a);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdn
