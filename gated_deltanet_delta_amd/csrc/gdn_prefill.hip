// Chunked (WY / UT-transform) prefill of the gated delta rule on gfx950.
//
// Inside a chunk of n <= 64 tokens of one sequence, with cumulative log-gates
// G_r = sum_{j<=r} g_j and the state S at the chunk start (d_v x d_k):
//   L_rj = beta_r e^{G_r - G_j} (k_r . k_j)   for r > j (0 otherwise)
//   T    = (I + L)^{-1}                                      (unit lower triangular)
//   U    = T diag(beta) (V - diag(e^G) K S^T)               (the corrected writes u_r)
//   O    = diag(e^G) Q S^T + P U,  P_rj = e^{G_r - G_j} (q_r . k_j) for j <= r
//   S   <- e^{G_last} S + (diag(e^{G_last - G}) U)^T K
// This is an exact reorganisation of the token-by-token rule (it follows from
// unrolling S_r = alpha_r S_{r-1} + u_r k_r^T inside the chunk).  Every
// exponent is a difference G_r - G_j with r >= j (or G_r itself), so it is
// <= 0 and nothing overflows.
//
// Three kernels per call, in stream order:
//   plan:   one workgroup turns the device cu_seqlens into a chunk table
//           (chunks restart at every sequence start; the last one may be
//           partial) and validates slots and lengths -- no host sync;
//   chunk:  one workgroup per (chunk, k-head): conv + SiLU + L2 norm of the
//           chunk's q, k (and v of the k-head's v-heads), gates and their
//           cumulative sums, A = K K^T and B = Q K^T on fp32 MFMA, then per
//           v-head L, the inverse T by forward substitution (one lane per
//           column, fp32), and P.  Everything goes to the workspace;
//   state:  one workgroup per (sequence, v-head, block of d_v rows) walks the
//           sequence's chunks in order with its fp32 state block resident in
//           MFMA accumulators and computes U, O and the next state with bf16
//           MFMA (fp32 MFMA for fp32 inputs).  It then writes the final state
//           and the conv history back to the sequence's slot.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kC = kChunk;   // 64 tokens per chunk
constexpr int kMaxGroup = 8; // v-heads per k-head supported by the chunk kernel

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int prefill_max_chunks(int n_tokens, int n_seqs) { return (n_tokens + kC - 1) / kC + n_seqs; }

PrefillLayout prefill_layout(int Hk, int Hv, int D, bool bf16, int maxc, int S) {
  const size_t es = bf16 ? 2 : 4;
  PrefillLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  const size_t mc = static_cast<size_t>(maxc);
  L.q = take(mc * Hk * kC * D * es);
  L.k = take(mc * Hk * kC * D * es);
  L.kt = take(mc * Hk * D * kC * es);
  L.v = take(mc * Hv * kC * D * es);
  L.t = take(mc * Hv * kC * kC * es);
  L.p = take(mc * Hv * kC * kC * es);
  L.g = take(mc * Hv * kC * 4);
  L.beta = take(mc * Hv * kC * 4);
  L.chunk_tab = take(mc * 4 * 4);
  L.seq_tab = take(static_cast<size_t>(S) * 8 * 4);
  L.counters = take(256);
  L.total = off;
  return L;
}

// Sequence table entry (int32 x 8).
enum { SQ_FIRST = 0, SQ_NCHUNK, SQ_POS0, SQ_FLAGS, SQ_SLOT, SQ_START, SQ_LEN, SQ_PAD };
enum { SQF_VALID = 1, SQF_INIT = 2 };

template <typename T>
__device__ __forceinline__ T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---------------------------------------------------------------------------
// plan: chunk table from cu_seqlens
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(PrefillArgs A, PrefillLayout L) {
  int32_t* ctab = ws_ptr<int32_t>(A.workspace, L.chunk_tab);
  int32_t* stab = ws_ptr<int32_t>(A.workspace, L.seq_tab);
  int32_t* cnt = ws_ptr<int32_t>(A.workspace, L.counters);
  __shared__ int s_total;
  if (threadIdx.x == 0) {
    const int S = A.n_seqs;
    bool ok = A.cu_seqlens[0] == 0 && A.cu_seqlens[S] == A.n_tokens;
    int bad_code = ok ? 0 : GDN_DEV_BAD_SEQLENS;
    int total = 0;
    for (int s = 0; s < S; ++s) {
      const int st = A.cu_seqlens[s];
      const int len = A.cu_seqlens[s + 1] - st;
      const int slot = A.slot[s];
      if (len < 0 || st < 0) { ok = false; if (!bad_code) bad_code = GDN_DEV_BAD_SEQLENS; }
      if (slot < 0 || slot >= A.n_slots) { ok = false; if (!bad_code) bad_code = GDN_DEV_BAD_SLOT; }
      const int nc = len > 0 ? (len + kC - 1) / kC : 0;
      const int init = A.has_init[s] != 0;
      int32_t* e = stab + 8 * s;
      e[SQ_FIRST] = total;
      e[SQ_NCHUNK] = nc;
      e[SQ_POS0] = (init && A.W > 0 && ok) ? static_cast<int32_t>(static_cast<uint32_t>(A.conv_pos[slot]) >> kPosShift) : 0;
      e[SQ_FLAGS] = SQF_VALID | (init ? SQF_INIT : 0);
      e[SQ_SLOT] = slot;
      e[SQ_START] = st;
      e[SQ_LEN] = len;
      e[SQ_PAD] = 0;
      total += nc > 0 ? nc : 0;
    }
    if (!ok) {
      report_error(A.dev_err, bad_code);
      for (int s = 0; s < S; ++s) stab[8 * s + SQ_FLAGS] = 0;
      total = 0;
    }
    if (total > A.max_chunks) total = 0;  // cannot happen for a valid partition
    cnt[0] = total;
    s_total = total;
  }
  __syncthreads();
  const int total = s_total;
  for (int c = threadIdx.x; c < total; c += blockDim.x) {
    int lo = 0, hi = A.n_seqs - 1;  // last s with first <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (stab[8 * mid + SQ_FIRST] <= c) lo = mid; else hi = mid - 1;
    }
    // sequences after the one holding c start beyond c, so lo holds c
    const int s = lo;
    const int i = c - stab[8 * s + SQ_FIRST];
    const int len = stab[8 * s + SQ_LEN];
    ctab[4 * c + 0] = s;
    ctab[4 * c + 1] = stab[8 * s + SQ_START] + i * kC;
    ctab[4 * c + 2] = min(kC, len - i * kC);
    ctab[4 * c + 3] = 0;
  }
}

// ---------------------------------------------------------------------------
// chunk: front end, gates, K K^T / Q K^T, inverse T, P
// ---------------------------------------------------------------------------
template <int D>
struct ChunkSmem {
  static constexpr int QK_LD = 2 * D + 1;              // q in [0,D), k in [D,2D)
  static constexpr int QK = kC * QK_LD;
  static constexpr int LM = 4 * kC * kC;               // up to 4 v-heads' L matrices
  static constexpr int UNION = QK > LM ? QK : LM;
  static constexpr int AB_LD = kC + 1;
  static constexpr int TOTAL = UNION + 2 * kC * AB_LD + 2 * kMaxGroup * kC + 2 * kC;
  static constexpr size_t BYTES = static_cast<size_t>(TOTAL) * 4;
};

template <bool BF16>
__device__ __forceinline__ void ws_store(void* base, size_t i, float v) {
  if constexpr (BF16) static_cast<uint16_t*>(base)[i] = f32_to_bf16_bits(v);
  else static_cast<float*>(base)[i] = v;
}

// Sliding-window causal conv of one channel over the chunk's tokens.
// Writes y(r) for r < len through `emit(r, y)`, zeros after.
template <bool BF16, typename Emit>
__device__ __forceinline__ void conv_chunk_channel(const PrefillArgs& A, int c, int t0, int len,
                                                   int seq_start, uint32_t pos0, bool init,
                                                   int slot, Emit emit) {
  const int W = A.W, C = A.C, R = A.R;
  // Fixed-size register arrays indexed with compile-time indices only.
  float hist[3] = {0.f, 0.f, 0.f};
  float w[3] = {0.f, 0.f, 0.f};
  const float wlast = W > 0 ? A.conv_w[c * W + W - 1] : 0.f;
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < W - 1) w[t] = A.conv_w[c * W + t];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    if (i < W - 1) {
      const int tt = t0 - (W - 1) + i;
      float v = 0.f;
      if (tt >= seq_start) {
        v = load_in<BF16>(A.x, static_cast<size_t>(tt) * C + c);
      } else if (init) {
        const int rel = tt - seq_start;  // -(W-1) .. -1
        v = A.conv_state[(static_cast<size_t>(slot) * R + ring_row(pos0 + static_cast<uint32_t>(rel), R)) * C + c];
      }
      hist[i] = v;
    }
  }
  for (int r = 0; r < kC; ++r) {
    float y = 0.f;
    if (r < len) {
      const float xin = load_in<BF16>(A.x, static_cast<size_t>(t0 + r) * C + c);
      if (W == 0) {
        y = xin;
      } else {
        // taps oldest first, the last one on the current token (same order as the step kernels)
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 3; ++t)
          if (t < W - 1) acc = fmaf(w[t], hist[t], acc);
        acc = fmaf(wlast, xin, acc);
        y = silu_f(acc);
        if (W == 4) { hist[0] = hist[1]; hist[1] = hist[2]; hist[2] = xin; }
        else if (W == 3) { hist[0] = hist[1]; hist[1] = xin; }
        else if (W == 2) { hist[0] = xin; }
      }
    }
    emit(r, y);
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void chunk_kernel(PrefillArgs A, PrefillLayout Lay) {
  using Sm = ChunkSmem<D>;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* qk = smem;                              // [64][2D+1]   (phase 1)
  float* Lm = smem;                              // [4][64][64]  (phase 2, reuses qk)
  float* Am = smem + Sm::UNION;                  // [64][65]  K K^T
  float* Bm = Am + kC * Sm::AB_LD;               // [64][65]  Q K^T
  float* gcum = Bm + kC * Sm::AB_LD;             // [G][64]
  float* bet = gcum + kMaxGroup * kC;            // [G][64]
  float* inv = bet + kMaxGroup * kC;             // [2][64]

  const int chunk = blockIdx.x;
  const int kh = blockIdx.y;
  const int n_chunks = ws_ptr<int32_t>(A.workspace, Lay.counters)[0];
  if (chunk >= n_chunks) return;
  const int32_t* ce = ws_ptr<int32_t>(A.workspace, Lay.chunk_tab) + 4 * chunk;
  const int s = ce[0], t0 = ce[1], len = ce[2];
  const int32_t* se = ws_ptr<int32_t>(A.workspace, Lay.seq_tab) + 8 * s;
  const bool init = (se[SQ_FLAGS] & SQF_INIT) != 0;
  const uint32_t pos0 = static_cast<uint32_t>(se[SQ_POS0]);
  const int slot = se[SQ_SLOT];
  const int seq_start = se[SQ_START];
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- q, k channels of this k-head: conv + SiLU into LDS ----
  for (int cc = tid; cc < 2 * D; cc += blockDim.x) {
    const int c = cc < D ? kh * D + cc : Hk * D + kh * D + (cc - D);
    conv_chunk_channel<BF16>(A, c, t0, len, seq_start, pos0, init, slot,
                             [&](int r, float y) { qk[r * Sm::QK_LD + cc] = y; });
  }
  // ---- v channels of the k-head's v-heads: straight to the workspace ----
  for (int cc = tid; cc < G * D; cc += blockDim.x) {
    const int h = kh * G + cc / D;
    const int dv = cc % D;
    const int c = 2 * Hk * D + h * D + dv;
    void* vb = static_cast<char*>(A.workspace) + Lay.v;
    const size_t base = (static_cast<size_t>(chunk) * Hv + h) * kC * D + dv;
    conv_chunk_channel<BF16>(A, c, t0, len, seq_start, pos0, init, slot,
                             [&](int r, float y) { ws_store<BF16>(vb, base + static_cast<size_t>(r) * D, y); });
  }
  // ---- gates: g = -softplus(a), beta = sigmoid(b), cumulative G ----
  if (tid < G) {
    const int h = kh * G + tid;
    float Gc = 0.f;
    float* wg = ws_ptr<float>(A.workspace, Lay.g) + (static_cast<size_t>(chunk) * Hv + h) * kC;
    float* wb = ws_ptr<float>(A.workspace, Lay.beta) + (static_cast<size_t>(chunk) * Hv + h) * kC;
    for (int r = 0; r < kC; ++r) {
      float g = 0.f, bb = 0.f;
      if (r < len) {
        const size_t i = static_cast<size_t>(t0 + r) * Hv + h;
        g = -softplus_f(load_in<BF16>(A.a, i));
        bb = sigmoid_f(load_in<BF16>(A.b, i));
      }
      Gc += g;
      gcum[tid * kC + r] = Gc;
      bet[tid * kC + r] = bb;
      wg[r] = Gc;
      wb[r] = bb;
    }
  }
  __syncthreads();

  // ---- L2 norm of q and k per token (fixed reduction order) ----
  const bool norm = (A.flags & GDN_FLAG_L2NORM_QK) != 0;
  for (int r = wave * 16; r < wave * 16 + 16; ++r) {
    float sq = 0.f, sk = 0.f;
    for (int d = lane; d < D; d += 64) {
      const float qv = qk[r * Sm::QK_LD + d];
      const float kv = qk[r * Sm::QK_LD + D + d];
      sq = fmaf(qv, qv, sq);
      sk = fmaf(kv, kv, sk);
    }
    sq = group_sum<64>(sq);
    sk = group_sum<64>(sk);
    if (lane == 0) {
      inv[r] = norm ? A.q_scale * (1.0f / sqrtf(sq + A.l2_eps)) : A.q_scale;
      inv[kC + r] = norm ? 1.0f / sqrtf(sk + A.l2_eps) : 1.0f;
    }
  }
  __syncthreads();
  for (int e = tid; e < kC * 2 * D; e += blockDim.x) {
    const int r = e / (2 * D), cc = e % (2 * D);
    qk[r * Sm::QK_LD + cc] *= inv[(cc >= D ? kC : 0) + r];
  }
  __syncthreads();

  // ---- q, k, k^T to the workspace ----
  {
    void* wq = static_cast<char*>(A.workspace) + Lay.q;
    void* wk = static_cast<char*>(A.workspace) + Lay.k;
    void* wkt = static_cast<char*>(A.workspace) + Lay.kt;
    const size_t base = (static_cast<size_t>(chunk) * Hk + kh) * kC * D;
    for (int e = tid; e < kC * D; e += blockDim.x) {
      const int r = e / D, d = e % D;
      ws_store<BF16>(wq, base + e, qk[r * Sm::QK_LD + d]);
      ws_store<BF16>(wk, base + e, qk[r * Sm::QK_LD + D + d]);
      const int d2 = e / kC, r2 = e % kC;
      ws_store<BF16>(wkt, base + e, qk[r2 * Sm::QK_LD + D + d2]);
    }
  }

  // ---- A = K K^T and B = Q K^T (lower triangles incl. diagonal), fp32 MFMA ----
  // 16x16x4 f32 MFMA: lane l supplies A[l%16][l/16] and B[l/16][l%16] and
  // receives D[4*(l/16)+i][l%16], i = 0..3.
  for (int task = wave; task < 20; task += 4) {
    const int which = task / 10;  // 0: K K^T, 1: Q K^T
    int t = task % 10, ti = 0;
    while (t > ti) { t -= ti + 1; ++ti; }
    const int tj = t;
    const float* lhs = qk + (which == 0 ? D : 0);
    const float* rhs = qk + D;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int ra = ti * 16 + (lane & 15), rb = tj * 16 + (lane & 15), kk = lane >> 4;
    for (int k0 = 0; k0 < D; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(lhs[ra * Sm::QK_LD + k0 + kk],
                                                 rhs[rb * Sm::QK_LD + k0 + kk], acc, 0, 0, 0);
    float* out = which == 0 ? Am : Bm;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(ti * 16 + (lane >> 4) * 4 + i) * Sm::AB_LD + tj * 16 + (lane & 15)] = acc[i];
  }
  __syncthreads();

  // ---- per v-head: L (LDS), P (workspace), T = (I+L)^{-1} (workspace) ----
  void* wt = static_cast<char*>(A.workspace) + Lay.t;
  void* wp = static_cast<char*>(A.workspace) + Lay.p;
  for (int hg0 = 0; hg0 < G; hg0 += 4) {
    const int nh = min(4, G - hg0);
    for (int e = tid; e < nh * kC * kC; e += blockDim.x) {
      const int i = e / (kC * kC), r = (e / kC) % kC, j = e % kC;
      const float* gc = gcum + (hg0 + i) * kC;
      Lm[e] = j < r ? bet[(hg0 + i) * kC + r] * expf(gc[r] - gc[j]) * Am[r * Sm::AB_LD + j] : 0.f;
      const float pv = j <= r ? expf(gc[r] - gc[j]) * Bm[r * Sm::AB_LD + j] : 0.f;
      const int h = kh * G + hg0 + i;
      ws_store<BF16>(wp, (static_cast<size_t>(chunk) * Hv + h) * kC * kC + r * kC + j, pv);
    }
    __syncthreads();
    if (wave < nh) {
      // Forward substitution for column `lane` of T: T[r][c] = d_rc - sum_{j<r} L[r][j] T[j][c].
      const float* Lw = Lm + wave * kC * kC;
      float t[kC];
#pragma unroll
      for (int r = 0; r < kC; ++r) {
        float acc = (r == lane) ? 1.0f : 0.0f;
        const float4* Lr = reinterpret_cast<const float4*>(Lw + r * kC);
#pragma unroll
        for (int j4 = 0; j4 < (r + 3) / 4; ++j4) {
          const float4 l4 = Lr[j4];
          if (4 * j4 + 0 < r) acc = fmaf(-l4.x, t[4 * j4 + 0], acc);
          if (4 * j4 + 1 < r) acc = fmaf(-l4.y, t[4 * j4 + 1], acc);
          if (4 * j4 + 2 < r) acc = fmaf(-l4.z, t[4 * j4 + 2], acc);
          if (4 * j4 + 3 < r) acc = fmaf(-l4.w, t[4 * j4 + 3], acc);
        }
        t[r] = acc;
      }
      const int h = kh * G + hg0 + wave;
      const size_t base = (static_cast<size_t>(chunk) * Hv + h) * kC * kC;
#pragma unroll
      for (int r = 0; r < kC; ++r) ws_store<BF16>(wt, base + r * kC + lane, t[r]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// state: sequential chunk loop per (sequence, v-head, d_v block)
// ---------------------------------------------------------------------------
template <bool BF16>
struct Mma;

// 16x16x32 bf16 MFMA: lane l supplies A[l%16][8*(l/16) + 0..7] and
// B[8*(l/16) + 0..7][l%16]; it receives D[4*(l/16) + i][l%16], i = 0..3.
template <>
struct Mma<true> {
  using E = uint16_t;
  using Op = bf16x8_t;
  static constexpr int KSTEP = 32;
  static constexpr int KPL = 8;
  static constexpr int PAD = 8;
  __device__ static Op load(const E* p) { return *reinterpret_cast<const Op*>(p); }
  __device__ static f32x4_t mma(Op a, Op b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static E cvt(float f) { return f32_to_bf16_bits(f); }
  __device__ static float back(E e) { return bf16_bits_to_f32(e); }
};

// 16x16x4 f32 MFMA: lane l supplies A[l%16][l/16] and B[l/16][l%16].
template <>
struct Mma<false> {
  using E = float;
  using Op = float;
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  static constexpr int PAD = 4;
  __device__ static Op load(const E* p) { return *p; }
  __device__ static f32x4_t mma(Op a, Op b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static E cvt(float f) { return f; }
  __device__ static float back(E e) { return e; }
};

template <int D>
struct StateShape {
  static constexpr int DVT = D >= 64 ? 32 : 16;        // d_v rows per workgroup
  static constexpr int NDT = DVT / 16;                 // 16-row tiles of the block
  static constexpr int NKT = D / 16;                   // 16-column tiles of d_k
  static constexpr int NS = (NDT * NKT + 3) / 4;       // state tiles per wave
};

// Operand of a 16-row tile at (row0, k0) of a row-major matrix with leading dimension ld.
// KLEN is the length of the contracted dimension when it is shorter than one
// MFMA k-step (d = 16 with the 32-deep bf16 MFMA): lanes whose k-range lies
// beyond it supply zeros and read nothing.
template <bool BF16, int KLEN = 1 << 30>
__device__ __forceinline__ typename Mma<BF16>::Op op_at(const typename Mma<BF16>::E* m, int ld,
                                                        int row0, int k0, int lane) {
  using M = Mma<BF16>;
  const int kk = k0 + (lane >> 4) * M::KPL;
  if constexpr (KLEN < M::KSTEP) {
    if (kk >= KLEN) return typename M::Op{};
  }
  return M::load(m + static_cast<size_t>(row0 + (lane & 15)) * ld + kk);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void state_kernel(PrefillArgs A, PrefillLayout Lay) {
  using M = Mma<BF16>;
  using E = typename M::E;
  using Sh = StateShape<D>;
  constexpr int DVT = Sh::DVT, NDT = Sh::NDT, NKT = Sh::NKT, NS = Sh::NS;
  constexpr int SLD = D + M::PAD;       // S block [DVT][D]
  constexpr int TLD = kC + M::PAD;      // R, U, Ut blocks [DVT][64]
  __shared__ __attribute__((aligned(16))) E S_l[DVT * SLD];
  __shared__ __attribute__((aligned(16))) E R_l[DVT * TLD];
  __shared__ __attribute__((aligned(16))) E U_l[DVT * TLD];
  __shared__ __attribute__((aligned(16))) E Ut_l[DVT * TLD];
  __shared__ float g_l[2][kC];
  __shared__ float b_l[2][kC];

  const int s = blockIdx.x, h = blockIdx.y, dv0 = blockIdx.z * DVT;
  const int32_t* se = ws_ptr<int32_t>(A.workspace, Lay.seq_tab) + 8 * s;
  if (!(se[SQ_FLAGS] & SQF_VALID)) return;
  const bool init = (se[SQ_FLAGS] & SQF_INIT) != 0;
  const int first = se[SQ_FIRST], nc = se[SQ_NCHUNK], slot = se[SQ_SLOT];
  const int seq_start = se[SQ_START], len = se[SQ_LEN];
  const uint32_t pos0 = static_cast<uint32_t>(se[SQ_POS0]);
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk, kh = h / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* ctab = ws_ptr<int32_t>(A.workspace, Lay.chunk_tab);
  const E* wq = ws_ptr<const E>(A.workspace, Lay.q);
  const E* wk = ws_ptr<const E>(A.workspace, Lay.k);
  const E* wkt = ws_ptr<const E>(A.workspace, Lay.kt);
  const E* wv = ws_ptr<const E>(A.workspace, Lay.v);
  const E* wT = ws_ptr<const E>(A.workspace, Lay.t);
  const E* wP = ws_ptr<const E>(A.workspace, Lay.p);
  const float* wg = ws_ptr<const float>(A.workspace, Lay.g);
  const float* wb = ws_ptr<const float>(A.workspace, Lay.beta);

  // ---- the state block in accumulators (fp32) and in LDS (operand type) ----
  float* Sglob = A.state + (static_cast<size_t>(slot) * Hv + h) * D * D;
  f32x4_t Sacc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int tt = wave + 4 * i;
    Sacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (tt < NDT * NKT) {
      const int dvt = tt / NKT, dkt = tt % NKT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dv = dvt * 16 + (lane >> 4) * 4 + e, dk = dkt * 16 + (lane & 15);
        const float v = init ? Sglob[static_cast<size_t>(dv0 + dv) * D + dk] : 0.f;
        Sacc[i][e] = v;
        S_l[dv * SLD + dk] = M::cvt(v);
      }
    }
  }

  const int tok = 16 * wave + (lane & 15);   // this lane's token column in steps 1-4
  for (int ci = 0; ci < nc; ++ci) {
    const int chunk = first + ci;
    const int t0 = ctab[4 * chunk + 1], clen = ctab[4 * chunk + 2];
    const int buf = ci & 1;
    if (tid < kC) {
      g_l[buf][tid] = wg[(static_cast<size_t>(chunk) * Hv + h) * kC + tid];
      b_l[buf][tid] = wb[(static_cast<size_t>(chunk) * Hv + h) * kC + tid];
    }
    __syncthreads();  // B0: S_l and gates ready; U_l, Ut_l free

    const E* Kc = wk + (static_cast<size_t>(chunk) * Hk + kh) * kC * D;
    const E* Qc = wq + (static_cast<size_t>(chunk) * Hk + kh) * kC * D;
    const E* KTc = wkt + (static_cast<size_t>(chunk) * Hk + kh) * D * kC;
    const E* Vc = wv + (static_cast<size_t>(chunk) * Hv + h) * kC * D;
    const E* Tc = wT + (static_cast<size_t>(chunk) * Hv + h) * kC * kC;
    const E* Pc = wP + (static_cast<size_t>(chunk) * Hv + h) * kC * kC;
    const float eG = expf(g_l[buf][tok]);
    const float bt = b_l[buf][tok];

    // steps 1 and 4a: X^T = S K^T and Y^T = S Q^T for this wave's 16 tokens;
    // step 2: R^T = (V^T - X^T diag(e^G)) diag(beta) -> LDS
    f32x4_t Y[NDT];
#pragma unroll
    for (int dvt = 0; dvt < NDT; ++dvt) {
      f32x4_t X = {0.f, 0.f, 0.f, 0.f};
      f32x4_t Yt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += M::KSTEP) {
        const auto a = op_at<BF16, D>(S_l, SLD, dvt * 16, k0, lane);
        X = M::mma(a, op_at<BF16, D>(Kc, D, 16 * wave, k0, lane), X);
        Yt = M::mma(a, op_at<BF16, D>(Qc, D, 16 * wave, k0, lane), Yt);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dv = dvt * 16 + (lane >> 4) * 4 + e;
        const float vv = M::back(Vc[static_cast<size_t>(tok) * D + dv0 + dv]);
        R_l[dv * TLD + tok] = M::cvt(bt * (vv - eG * X[e]));
        Y[dvt][e] = eG * Yt[e];
      }
    }
    __syncthreads();  // B1: R_l complete

    // step 3: U^T = R^T T^T (T lower triangular: j < 16*wave + 16)
    const int kend = 16 * wave + 16;
    const float dec = expf(g_l[buf][kC - 1] - g_l[buf][tok]);
#pragma unroll
    for (int dvt = 0; dvt < NDT; ++dvt) {
      f32x4_t U = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < kend; k0 += M::KSTEP)
        U = M::mma(op_at<BF16>(R_l, TLD, dvt * 16, k0, lane), op_at<BF16>(Tc, kC, 16 * wave, k0, lane), U);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dv = dvt * 16 + (lane >> 4) * 4 + e;
        U_l[dv * TLD + tok] = M::cvt(U[e]);
        Ut_l[dv * TLD + tok] = M::cvt(U[e] * dec);
      }
    }
    __syncthreads();  // B2: U_l, Ut_l complete

    // step 4b: O^T = Y^T + U^T P^T (P lower triangular), written for valid tokens
#pragma unroll
    for (int dvt = 0; dvt < NDT; ++dvt) {
      f32x4_t O = Y[dvt];
      for (int k0 = 0; k0 < kend; k0 += M::KSTEP)
        O = M::mma(op_at<BF16>(U_l, TLD, dvt * 16, k0, lane), op_at<BF16>(Pc, kC, 16 * wave, k0, lane), O);
      if (tok < clen) {
        const size_t ob = (static_cast<size_t>(t0 + tok) * Hv + h) * D + dv0 + dvt * 16 + (lane >> 4) * 4;
        if constexpr (BF16) {
          uint2 pk;
          pk.x = static_cast<uint32_t>(f32_to_bf16_bits(O[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(O[1])) << 16);
          pk.y = static_cast<uint32_t>(f32_to_bf16_bits(O[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(O[3])) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(A.o) + ob) = pk;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(A.o) + ob) = make_float4(O[0], O[1], O[2], O[3]);
        }
      }
    }

    // step 5: S <- e^{G_last} S + Ut^T K
    const float eGl = expf(g_l[buf][kC - 1]);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int tt = wave + 4 * i;
      if (tt < NDT * NKT) {
        const int dvt = tt / NKT, dkt = tt % NKT;
        f32x4_t acc = Sacc[i] * eGl;
#pragma unroll
        for (int k0 = 0; k0 < kC; k0 += M::KSTEP)
          acc = M::mma(op_at<BF16>(Ut_l, TLD, dvt * 16, k0, lane), op_at<BF16>(KTc, kC, dkt * 16, k0, lane), acc);
        Sacc[i] = acc;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S_l[(dvt * 16 + (lane >> 4) * 4 + e) * SLD + dkt * 16 + (lane & 15)] = M::cvt(acc[e]);
      }
    }
  }

  // ---- final state back to the slot ----
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int tt = wave + 4 * i;
    if (tt < NDT * NKT) {
      const int dvt = tt / NKT, dkt = tt % NKT;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dv = dvt * 16 + (lane >> 4) * 4 + e, dk = dkt * 16 + (lane & 15);
        Sglob[static_cast<size_t>(dv0 + dv) * D + dk] = Sacc[i][e];
      }
    }
  }

  // ---- conv history: the last W-1 inputs go to ring rows pos_end-1 .. pos_end-W+1 ----
  if (A.W > 0) {
    const int W = A.W, C = A.C, R = A.R;
    const uint32_t pos_end = (init ? pos0 : 0u) + static_cast<uint32_t>(len);
    float* ring = A.conv_state + static_cast<size_t>(slot) * R * C;
    auto put = [&](int c) {
      for (int i = 1; i < W; ++i) {
        const int rel = len - i;
        float* dst = ring + static_cast<size_t>(ring_row(pos_end - i, R)) * C + c;
        if (rel >= 0) *dst = load_in<BF16>(A.x, static_cast<size_t>(seq_start + rel) * C + c);
        else if (!init) *dst = 0.f;
      }
    };
    if (h % G == 0 && blockIdx.z == 0)
      for (int cc = tid; cc < 2 * D; cc += blockDim.x) put(cc < D ? kh * D + cc : Hk * D + kh * D + (cc - D));
    for (int cc = tid; cc < DVT; cc += blockDim.x) put(2 * Hk * D + h * D + dv0 + cc);
    if (h == 0 && blockIdx.z == 0 && tid == 0)
      A.conv_pos[slot] = static_cast<int32_t>(pos_end << kPosShift);
  }
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------
template <int D, bool BF16>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const PrefillLayout L = prefill_layout(a.Hk, a.Hv, D, BF16, a.max_chunks, a.n_seqs);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, a, L);
  int e = static_cast<int>(hipGetLastError());
  if (e) return e;
  const size_t smem = ChunkSmem<D>::BYTES;
  e = static_cast<int>(hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_kernel<D, BF16>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(smem)));
  if (e) return e;
  if (a.max_chunks > 0) {
    hipLaunchKernelGGL((chunk_kernel<D, BF16>), dim3(a.max_chunks, a.Hk), dim3(256), smem, st, a, L);
    e = static_cast<int>(hipGetLastError());
    if (e) return e;
  }
  hipLaunchKernelGGL((state_kernel<D, BF16>), dim3(a.n_seqs, a.Hv, D / StateShape<D>::DVT), dim3(256), 0,
                     st, a, L);
  return static_cast<int>(hipGetLastError());
}

int launch_prefill(const PrefillArgs& a, bool bf16, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.D) {
    case 16: return bf16 ? launch_prefill_t<16, true>(a, s) : launch_prefill_t<16, false>(a, s);
    case 32: return bf16 ? launch_prefill_t<32, true>(a, s) : launch_prefill_t<32, false>(a, s);
    case 64: return bf16 ? launch_prefill_t<64, true>(a, s) : launch_prefill_t<64, false>(a, s);
    case 128: return bf16 ? launch_prefill_t<128, true>(a, s) : launch_prefill_t<128, false>(a, s);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace gdn
