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
//   chunk:  one workgroup per (chunk, k-head), all chunks in parallel: conv +
//           SiLU + L2 norm of the chunk's q, k and v, gates and their
//           cumulative sums, K K^T and Q K^T on MFMA, then per v-head L, the
//           inverse T and P.  Every matrix the next kernel multiplies is
//           written pre-packed in MFMA operand order (below), V already
//           scaled by beta, and the per-token gate factors precomputed;
//   chain:  one wave per (sequence, v-head, 16 rows of d_v) walks the
//           sequence's chunks in order.  It keeps its 16 x d_k slice of the
//           state, transposed, in MFMA accumulators and never leaves
//           registers: every product's result feeds the next product as its
//           B operand directly (the contraction order inside an MFMA is a
//           free permutation, so the A operand is packed in the permuted
//           order that matches the accumulator layout).  The waves of a
//           workgroup share the chunk's packed operands, staged into LDS
//           with direct global->LDS loads one chunk ahead.
//
// Packed operand tiles.  A 16 x SK sub-matrix (rows r, contraction index k;
// SK = 32 for the bf16 MFMA 16x16x32, 16 for four fp32 MFMA 16x16x4) is
// stored as 64 lanes x 16 bytes.  Lane (g = k%16 / 4) * 16 + r holds, in
// element e = (k / 16) * 4 + k % 4, the value at (r, k).  A 16x16
// accumulator tile holds rows 4g..4g+3 of column l%16 in lane l, so the
// accumulators of tiles (2s, 2s+1) (bf16) or tile s (fp32) form exactly the
// B operand that pairs with packed tile column s.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kC = kChunk;    // 64 tokens per chunk
constexpr int kMaxGroup = 8;  // v-heads per k-head
constexpr int kLd = kC + 1;   // row stride of 64x64 fp32 matrices in LDS
constexpr int kTileBytes = 1024;

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

template <bool BF16>
struct Pk {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int SK = BF16 ? 32 : 16;         // contraction length of one packed tile
  static constexpr int EPL = BF16 ? 8 : 4;          // elements per lane (16 bytes)
  static constexpr int VC_BYTES = 256 * sizeof(E);  // one 16x16 tile in accumulator layout
};

template <int D, bool BF16>
struct Geo {
  using P = Pk<BF16>;
  static constexpr int KSD = (D + P::SK - 1) / P::SK;  // packed tiles along d
  static constexpr int KSC = kC / P::SK;               // packed tiles along the chunk
  static constexpr int NT = D / 16;                    // 16-row tiles along d
  static constexpr int KA = 0;                         // K  as A (rows tok, k = d):   4 x KSD
  static constexpr int QA = 4 * KSD;                   // Q  as A:                     4 x KSD
  static constexpr int KTA = 8 * KSD;                  // K^T as A (rows d, k = tok): NT x KSC
  static constexpr int KQ_TILES = 8 * KSD + NT * KSC;
  static constexpr int TA = 0;                         // T as A (rows r, k = j):      4 x KSC
  static constexpr int PA = 4 * KSC;                   // P as A:                      4 x KSC
  static constexpr size_t VC_OFF = 8 * KSC * kTileBytes;            // V, accumulator layout [NT][4]
  // per-token factors: e^G, beta e^G, e^{G_last - G}, then e^{G_last} (4 x 64 floats)
  static constexpr size_t GATE_OFF = VC_OFF + NT * 4 * P::VC_BYTES;
  static constexpr size_t GATE_BYTES = 4 * kC * 4;
  static constexpr size_t KQ_BYTES = KQ_TILES * kTileBytes;
  static constexpr size_t HEAD_BYTES = GATE_OFF + GATE_BYTES;
};

int prefill_max_chunks(int n_tokens, int n_seqs) { return (n_tokens + kC - 1) / kC + n_seqs; }

template <int D, bool BF16>
static PrefillLayout layout_t(int Hk, int Hv, int maxc, int S) {
  using Gm = Geo<D, BF16>;
  PrefillLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  const size_t mc = static_cast<size_t>(maxc);
  L.kq_bytes = Gm::KQ_BYTES;
  L.head_bytes = Gm::HEAD_BYTES;
  L.kq = take(mc * Hk * Gm::KQ_BYTES);
  L.head = take(mc * Hv * Gm::HEAD_BYTES);
  L.chunk_tab = take(mc * 4 * 4);
  L.seq_tab = take(static_cast<size_t>(S) * 8 * 4);
  L.counters = take(256);
  L.total = off;
  return L;
}

PrefillLayout prefill_layout(int Hk, int Hv, int D, bool bf16, int maxc, int S) {
  switch (D) {
    case 16: return bf16 ? layout_t<16, true>(Hk, Hv, maxc, S) : layout_t<16, false>(Hk, Hv, maxc, S);
    case 32: return bf16 ? layout_t<32, true>(Hk, Hv, maxc, S) : layout_t<32, false>(Hk, Hv, maxc, S);
    case 64: return bf16 ? layout_t<64, true>(Hk, Hv, maxc, S) : layout_t<64, false>(Hk, Hv, maxc, S);
    default: return bf16 ? layout_t<128, true>(Hk, Hv, maxc, S) : layout_t<128, false>(Hk, Hv, maxc, S);
  }
}

// Sequence table entry (int32 x 8).
enum { SQ_FIRST = 0, SQ_NCHUNK, SQ_POS0, SQ_FLAGS, SQ_SLOT, SQ_START, SQ_LEN, SQ_PAD };
enum { SQF_VALID = 1, SQF_INIT = 2 };

template <typename T>
__device__ __forceinline__ T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Workgroup barrier that orders LDS traffic only: global loads issued before
// it stay in flight (a full __syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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
      total += nc;
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
    int lo = 0, hi = A.n_seqs - 1;  // last s with first <= c holds c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (stab[8 * mid + SQ_FIRST] <= c) lo = mid; else hi = mid - 1;
    }
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
// shared MFMA helpers
// ---------------------------------------------------------------------------
// 16x16x4 fp32 MFMA: lane l supplies A[l%16][l/16] and B[l/16][l%16] and
// receives D[4*(l/16)+i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 MFMA: lane l supplies 8 k-values of row l%16 of A and of
// column l%16 of B (the same 8 k-values: group l/16), receives as above.
__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One packed super-step: A is a packed tile (16 bytes of this lane), B is
// made of accumulator tiles of a previous product.
template <bool BF16>
struct Chain;

template <>
struct Chain<true> {
  using Bop = bf16x8_t;
  __device__ static Bop bop(const f32x4_t& t0, const f32x4_t& t1) {
    Bop b;
    b[0] = static_cast<__bf16>(t0[0]); b[1] = static_cast<__bf16>(t0[1]);
    b[2] = static_cast<__bf16>(t0[2]); b[3] = static_cast<__bf16>(t0[3]);
    b[4] = static_cast<__bf16>(t1[0]); b[5] = static_cast<__bf16>(t1[1]);
    b[6] = static_cast<__bf16>(t1[2]); b[7] = static_cast<__bf16>(t1[3]);
    return b;
  }
  __device__ static f32x4_t step(uint4 a, const Bop& b, f32x4_t c) {
    return mfma32(__builtin_bit_cast(bf16x8_t, a), b, c);
  }
};

template <>
struct Chain<false> {
  using Bop = f32x4_t;
  __device__ static Bop bop(const f32x4_t& t0, const f32x4_t&) { return t0; }
  __device__ static f32x4_t step(uint4 a, const Bop& b, f32x4_t c) {
    c = mfma4(__uint_as_float(a.x), b[0], c);
    c = mfma4(__uint_as_float(a.y), b[1], c);
    c = mfma4(__uint_as_float(a.z), b[2], c);
    return mfma4(__uint_as_float(a.w), b[3], c);
  }
};

// SiLU with the hardware exp and reciprocal (the front end runs it on every
// input of every token, so it is kept to five instructions).
__device__ __forceinline__ float silu_fast(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// acc += A (16x16, row-major at a, stride lda) * B (16x16, row-major at b, stride ldb); fp32.
__device__ __forceinline__ f32x4_t prod16(const float* a, int lda, const float* b, int ldb,
                                          f32x4_t acc, int lane) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = mfma4(a[(lane & 15) * lda + 4 * s + (lane >> 4)], b[(4 * s + (lane >> 4)) * ldb + (lane & 15)], acc);
  return acc;
}

__device__ __forceinline__ void store16(float* d, int ld, f32x4_t v, float sign, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) d[(4 * (lane >> 4) + i) * ld + (lane & 15)] = sign * v[i];
}

// In-place inverse of the unit lower-triangular I + L (64x64, L strictly lower,
// row stride kLd) by one wave: 16x16 diagonal blocks by forward substitution
// (lane = block x column), then the off-diagonal blocks level by level with
// fp32 MFMA:  [A 0; C B]^-1 = [A^-1 0; -B^-1 C A^-1  B^-1].
// tmp: 32 x 33 floats of scratch.
__device__ void invert_unit_lower64(float* Lt, float* tmp, int lane) {
  {
    const int bi = lane >> 4, c = lane & 15;
    float* Lb = Lt + 16 * bi * kLd + 16 * bi;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == c) ? 1.0f : 0.0f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc = fmaf(-Lb[r * kLd + j], t[j], acc);
      t[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Lb[r * kLd + c] = t[r];
  }
  // 32x32 level: T10 = -T11 (L10 T00) in both diagonal 32-blocks
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float* o = Lt + 32 * b * kLd + 32 * b;
    f32x4_t m = prod16(o + 16 * kLd, kLd, o, kLd, f32x4_t{0.f, 0.f, 0.f, 0.f}, lane);
    store16(tmp, 17, m, 1.0f, lane);
    f32x4_t r = prod16(o + 16 * kLd + 16, kLd, tmp, 17, f32x4_t{0.f, 0.f, 0.f, 0.f}, lane);
    store16(o + 16 * kLd, kLd, r, -1.0f, lane);
  }
  // 64x64 level: T_BA = -T_B (C T_A), 32x32 blocks; C is the lower-left block of L
  const float* C = Lt + 32 * kLd;
  const float* TA = Lt;
  const float* TB = Lt + 32 * kLd + 32;
  f32x4_t m2[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = ct; kt < 2; ++kt)  // T_A[kt][ct] = 0 for kt < ct
        acc = prod16(C + 16 * rt * kLd + 16 * kt, kLd, TA + 16 * kt * kLd + 16 * ct, kLd, acc, lane);
      m2[rt][ct] = acc;
    }
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) store16(tmp + 16 * rt * 33 + 16 * ct, 33, m2[rt][ct], 1.0f, lane);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt <= rt; ++kt)  // T_B[rt][kt] = 0 for kt > rt
        acc = prod16(TB + 16 * rt * kLd + 16 * kt, kLd, tmp + 16 * kt * 33 + 16 * ct, 33, acc, lane);
      store16(Lt + (32 + 16 * rt) * kLd + 16 * ct, kLd, acc, -1.0f, lane);
    }
}

template <bool BF16>
__device__ __forceinline__ typename Pk<BF16>::E to_e(float v) {
  if constexpr (BF16) return f32_to_bf16_bits(v);
  else return v;
}

// 16 bytes of a packed lane from the EPL values f(0..EPL-1).
template <bool BF16, typename F>
__device__ __forceinline__ uint4 pack_lane(F f) {
  if constexpr (BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16_bits(f(2 * i))) |
             (static_cast<uint32_t>(f32_to_bf16_bits(f(2 * i + 1))) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__float_as_uint(f(0)), __float_as_uint(f(1)), __float_as_uint(f(2)), __float_as_uint(f(3)));
  }
}

// ---------------------------------------------------------------------------
// chunk: front end, gates, K K^T / Q K^T, inverse T, P  (8 waves)
// ---------------------------------------------------------------------------
constexpr int kChunkThreads = 512;

template <int D, bool BF16>
struct ChunkSmem {
  static constexpr int QK_LD = 2 * D + 1;               // q in [0,D), k in [D,2D)
  static constexpr int QK = (kC * QK_LD > 4 * kC * kLd) ? kC * QK_LD : 4 * kC * kLd;  // qk, then L/T
  static constexpr int PKT = BF16 ? 3 * 4 * Geo<D, BF16>::KSD * kTileBytes / 4 : 0;   // hi, lo, q tiles
  static constexpr int PK = PKT > 4 * 32 * 33 ? PKT : 4 * 32 * 33;                   // then inverse scratch
  static constexpr int AB = 2 * kC * kLd;
  static constexpr int MISC = 2 * kMaxGroup * kC + 2 * kC;
  static constexpr size_t BYTES = static_cast<size_t>(QK + PK + AB + MISC) * 4;
};

template <int D, bool BF16>
__global__ __launch_bounds__(kChunkThreads) void chunk_kernel(PrefillArgs A, PrefillLayout Lay) {
  using P = Pk<BF16>;
  using Gm = Geo<D, BF16>;
  using Sm = ChunkSmem<D, BF16>;
  using E = typename P::E;
  constexpr int VE = 16 / sizeof(E);            // channels per 16-byte input vector
  constexpr int KSD = Gm::KSD, KSC = Gm::KSC, NT = Gm::NT;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* qk = smem;                               // [64][2D+1] raw conv outputs of q | k
  float* Lt = smem;                               // [4][64][65] L -> T   (per-head phase)
  uint4* pk = reinterpret_cast<uint4*>(smem + Sm::QK);  // packed k_hi, k_lo, q tiles (bf16 only)
  float* tmpw = smem + Sm::QK;                    // [4][32][33] inverse scratch (per-head phase)
  float* Am = smem + Sm::QK + Sm::PK;             // [64][65] K K^T (normalised)
  float* Bm = Am + kC * kLd;                      // [64][65] Q K^T (normalised, q_scale)
  float* gcum = Bm + kC * kLd;                    // [8][64]
  float* bet = gcum + kMaxGroup * kC;             // [8][64]
  float* inv = bet + kMaxGroup * kC;              // [2][64]  q and k scale factors

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
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk, C = A.C, R = A.R, W = A.W;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NCH = (2 + G) * D;                    // channels of this k-head: q | k | v of its v-heads
  const E* x = static_cast<const E*>(A.x);
  char* kqb = static_cast<char*>(A.workspace) + Lay.kq + (static_cast<size_t>(chunk) * Hk + kh) * Gm::KQ_BYTES;
  auto headb = [&](int h) {
    return static_cast<char*>(A.workspace) + Lay.head + (static_cast<size_t>(chunk) * Hv + h) * Gm::HEAD_BYTES;
  };
  auto xchan = [&](int cc) {
    return cc < D ? kh * D + cc : (cc < 2 * D ? Hk * D + kh * D + (cc - D) : 2 * Hk * D + kh * G * D + (cc - 2 * D));
  };

  // ---- gates: one wave per v-head, lane = token, fixed-order inclusive scan ----
  for (int hi = wave; hi < G; hi += kChunkThreads / 64) {
    const int h = kh * G + hi;
    float g = 0.f, bb = 0.f;
    if (lane < len) {
      const size_t i = static_cast<size_t>(t0 + lane) * Hv + h;
      g = -softplus_f(load_in<BF16>(A.a, i));
      bb = sigmoid_f(load_in<BF16>(A.b, i));
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float up = __shfl_up(g, off, 64);
      if (lane >= off) g += up;
    }
    gcum[hi * kC + lane] = g;
    bet[hi * kC + lane] = bb;
    const float glast = __shfl(g, 63, 64);
    const float eg = __expf(g);
    float* gw = reinterpret_cast<float*>(headb(h) + Gm::GATE_OFF);
    gw[lane] = eg;
    gw[kC + lane] = bb * eg;
    gw[2 * kC + lane] = __expf(glast - g);
    gw[3 * kC + lane] = __expf(glast);
  }

  __syncthreads();  // betas are in LDS: V is stored pre-scaled by beta

  // ---- conv + SiLU: item = (VE channels, 16 tokens), the 19-row window in registers ----
  const int nvec = NCH / VE;
  for (int item = tid; item < 4 * nvec; item += kChunkThreads) {
    const int q = item / nvec, cc0 = (item - q * nvec) * VE;
    const int c0 = xchan(cc0);
    const int tq = 16 * q;                        // first token of this quarter
    // raw rows: tokens t0+tq-3 .. t0+tq+15 (row i <-> token t0+tq-3+i),
    // clamped into the sequence and the chunk so every load is valid
    uint4 raw[19];
#pragma unroll
    for (int i = 0; i < 19; ++i) {
      const int t = min(max(t0 + tq - 3 + i, seq_start), t0 + len - 1);
      raw[i] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t) * C + c0);
    }
    float w[VE][4];
    if (W == 4) {
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        const float4 w4 = *reinterpret_cast<const float4*>(A.conv_w + (c0 + v) * 4);
        w[v][0] = w4.x; w[v][1] = w4.y; w[v][2] = w4.z; w[v][3] = w4.w;
      }
    }
    auto elem = [&](const uint4& r, int v) -> float {
      if constexpr (BF16) {
        const uint32_t wv = (v >> 1) == 0 ? r.x : (v >> 1) == 1 ? r.y : (v >> 1) == 2 ? r.z : r.w;
        return __uint_as_float((v & 1) ? (wv & 0xffff0000u) : (wv << 16));
      } else {
        return __uint_as_float(v == 0 ? r.x : v == 1 ? r.y : v == 2 ? r.z : r.w);
      }
    };
    // the three rows before the quarter: x, or the ring / zero before the sequence
    float hist[VE][3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int t = t0 + tq - 3 + i;
#pragma unroll
      for (int v = 0; v < VE; ++v) hist[v][i] = elem(raw[i], v);
      if (t < seq_start) {
        if (init) {
          const float* rr = A.conv_state + (static_cast<size_t>(slot) * R +
                                            ring_row(pos0 + static_cast<uint32_t>(t - seq_start), R)) * C + c0;
#pragma unroll
          for (int v = 0; v < VE; ++v) hist[v][i] = rr[v];
        } else {
#pragma unroll
          for (int v = 0; v < VE; ++v) hist[v][i] = 0.f;
        }
      }
    }
    const bool is_v = cc0 >= 2 * D;
    const int hv = is_v ? (cc0 - 2 * D) / D : 0;  // v-head within the group
    const int dv0 = is_v ? (cc0 - 2 * D) % D : 0;
    E* vcb = reinterpret_cast<E*>(headb(kh * G + hv) + Gm::VC_OFF);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {              // 4 groups of 4 tokens
      float y[VE][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;                 // token within the quarter
        const bool valid = tq + r < len;
#pragma unroll
        for (int v = 0; v < VE; ++v) {
          const float xin = elem(raw[3 + r], v);
          float yy;
          if (W == 4) {
            float acc = w[v][0] * hist[v][0];
            acc = fmaf(w[v][1], hist[v][1], acc);
            acc = fmaf(w[v][2], hist[v][2], acc);
            acc = fmaf(w[v][3], xin, acc);
            yy = silu_fast(acc);
            hist[v][0] = hist[v][1]; hist[v][1] = hist[v][2]; hist[v][2] = xin;
          } else {
            yy = xin;
          }
          y[v][i] = valid ? yy : 0.f;
        }
      }
      if (!is_v) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < VE; ++v) qk[(tq + 4 * g4 + i) * Sm::QK_LD + cc0 + v] = y[v][i];
      } else {
        // accumulator layout: tile (dv/16, quarter q), lane g4*16 + dv%16, elements i;
        // stored as beta * v
        const float4 bq = *reinterpret_cast<const float4*>(bet + hv * kC + tq + 4 * g4);
#pragma unroll
        for (int v = 0; v < VE; ++v) {
          y[v][0] *= bq.x; y[v][1] *= bq.y; y[v][2] *= bq.z; y[v][3] *= bq.w;
        }
#pragma unroll
        for (int v = 0; v < VE; ++v) {
          const int dv = dv0 + v;
          E* dst = vcb + ((dv >> 4) * 4 + q) * 256 + (g4 * 16 + (dv & 15)) * 4;
          if constexpr (BF16) {
            uint2 pkd;
            pkd.x = static_cast<uint32_t>(f32_to_bf16_bits(y[v][0])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[v][1])) << 16);
            pkd.y = static_cast<uint32_t>(f32_to_bf16_bits(y[v][2])) | (static_cast<uint32_t>(f32_to_bf16_bits(y[v][3])) << 16);
            *reinterpret_cast<uint2*>(dst) = pkd;
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(y[v][0], y[v][1], y[v][2], y[v][3]);
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- L2 norm factors of q and k per token (fixed reduction order) ----
  const bool norm = (A.flags & GDN_FLAG_L2NORM_QK) != 0;
  for (int r = wave * 8; r < wave * 8 + 8; ++r) {
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
  auto qn = [&](int r, int d) { return qk[r * Sm::QK_LD + d] * inv[r]; };
  auto kn = [&](int r, int d) { return qk[r * Sm::QK_LD + D + d] * inv[kC + r]; };

  // ---- packed K, Q (rows tok, k = d) and K^T (rows d, k = tok) to the workspace ----
  // (bf16: also k_hi, k_lo, q tiles into LDS for the K K^T / Q K^T products)
  for (int u = tid; u < 4 * KSD * 64; u += kChunkThreads) {
    const int tile = u >> 6, ln = u & 63;
    const int mt = tile / KSD, ks = tile % KSD;
    const int row = 16 * mt + (ln & 15), g = ln >> 4;
    auto kof = [&](int e) { return ks * P::SK + (e >> 2) * 16 + 4 * g + (e & 3); };
    const uint4 kw = pack_lane<BF16>([&](int e) { const int k = kof(e); return k < D ? kn(row, k) : 0.f; });
    const uint4 qw = pack_lane<BF16>([&](int e) { const int k = kof(e); return k < D ? qn(row, k) : 0.f; });
    reinterpret_cast<uint4*>(kqb + (Gm::KA + tile) * kTileBytes)[ln] = kw;
    reinterpret_cast<uint4*>(kqb + (Gm::QA + tile) * kTileBytes)[ln] = qw;
    if constexpr (BF16) {
      const uint4 lw = pack_lane<BF16>([&](int e) {
        const int k = kof(e);
        if (k >= D) return 0.f;
        const float v = kn(row, k);
        return v - bf16_bits_to_f32(f32_to_bf16_bits(v));
      });
      pk[(0 * 4 * KSD + tile) * 64 + ln] = kw;
      pk[(1 * 4 * KSD + tile) * 64 + ln] = lw;
      pk[(2 * 4 * KSD + tile) * 64 + ln] = qw;
    }
  }
  for (int u = tid; u < NT * KSC * 64; u += kChunkThreads) {
    const int tile = u >> 6, ln = u & 63;
    const int mt = tile / KSC, ks = tile % KSC;
    const int dk = 16 * mt + (ln & 15), g = ln >> 4;
    const uint4 w4 = pack_lane<BF16>([&](int e) { return kn(ks * P::SK + (e >> 2) * 16 + 4 * g + (e & 3), dk); });
    reinterpret_cast<uint4*>(kqb + (Gm::KTA + tile) * kTileBytes)[ln] = w4;
  }
  __syncthreads();

  // ---- A = K K^T and B = Q K^T (lower 16x16 tiles incl. the diagonal) ----
  for (int task = wave; task < 20; task += kChunkThreads / 64) {
    const int which = task / 10;  // 0: K K^T, 1: Q K^T
    int t = task % 10, ti = 0;
    while (t > ti) { t -= ti + 1; ++ti; }
    const int tj = t;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
      // K K^T (which feeds the inverse) sums hi*hi + hi*lo + lo*hi for about
      // fp32 accuracy; Q K^T (stored as bf16) takes one product.  A packed
      // K tile is also the B operand of K^T (same lanes, same k order).
      const uint4* khi = pk;
      const uint4* klo = pk + 4 * KSD * 64;
      const uint4* qq = pk + 2 * 4 * KSD * 64;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, khi[(tj * KSD + ks) * 64 + lane]);
        if (which == 0) {
          const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, khi[(ti * KSD + ks) * 64 + lane]);
          const bf16x8_t al = __builtin_bit_cast(bf16x8_t, klo[(ti * KSD + ks) * 64 + lane]);
          const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, klo[(tj * KSD + ks) * 64 + lane]);
          acc = mfma32(ah, bh, acc);
          acc = mfma32(ah, bl, acc);
          acc = mfma32(al, bh, acc);
        } else {
          acc = mfma32(__builtin_bit_cast(bf16x8_t, qq[(ti * KSD + ks) * 64 + lane]), bh, acc);
        }
      }
    } else {
      const int ra = ti * 16 + (lane & 15), rb = tj * 16 + (lane & 15), kk = lane >> 4;
      for (int k0 = 0; k0 < D; k0 += 4) {
        const float av = which == 0 ? kn(ra, k0 + kk) : qn(ra, k0 + kk);
        acc = mfma4(av, kn(rb, k0 + kk), acc);
      }
    }
    float* out = which == 0 ? Am : Bm;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[(ti * 16 + (lane >> 4) * 4 + i) * kLd + tj * 16 + (lane & 15)] = acc[i];
  }
  __syncthreads();

  // ---- per v-head: L (LDS), P and T (packed, workspace) ----
  for (int hg0 = 0; hg0 < G; hg0 += 4) {
    const int nh = min(4, G - hg0);
    for (int e = tid; e < nh * kC * kC; e += kChunkThreads) {
      const int i = e / (kC * kC), r = (e / kC) % kC, j = e % kC;
      const float* gc = gcum + (hg0 + i) * kC;
      Lt[i * kC * kLd + r * kLd + j] = j < r ? bet[(hg0 + i) * kC + r] * __expf(gc[r] - gc[j]) * Am[r * kLd + j] : 0.f;
    }
    for (int u = tid; u < nh * 4 * KSC * 64; u += kChunkThreads) {
      const int i = u / (4 * KSC * 64), tile = (u >> 6) % (4 * KSC), ln = u & 63;
      const int mt = tile / KSC, ks = tile % KSC;
      const int r = 16 * mt + (ln & 15), g = ln >> 4;
      const float* gc = gcum + (hg0 + i) * kC;
      const uint4 w4 = pack_lane<BF16>([&](int e) {
        const int j = ks * P::SK + (e >> 2) * 16 + 4 * g + (e & 3);
        return j <= r ? __expf(gc[r] - gc[j]) * Bm[r * kLd + j] : 0.f;
      });
      reinterpret_cast<uint4*>(headb(kh * G + hg0 + i) + (Gm::PA + tile) * kTileBytes)[ln] = w4;
    }
    __syncthreads();
    if (wave < nh) invert_unit_lower64(Lt + wave * kC * kLd, tmpw + wave * 32 * 33, lane);
    __syncthreads();
    for (int u = tid; u < nh * 4 * KSC * 64; u += kChunkThreads) {
      const int i = u / (4 * KSC * 64), tile = (u >> 6) % (4 * KSC), ln = u & 63;
      const int mt = tile / KSC, ks = tile % KSC;
      const int r = 16 * mt + (ln & 15), g = ln >> 4;
      const float* Ti = Lt + i * kC * kLd;
      const uint4 w4 = pack_lane<BF16>([&](int e) { return Ti[r * kLd + ks * P::SK + (e >> 2) * 16 + 4 * g + (e & 3)]; });
      reinterpret_cast<uint4*>(headb(kh * G + hg0 + i) + (Gm::TA + tile) * kTileBytes)[ln] = w4;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// chain: sequential chunk loop, one wave per 16 rows of d_v
// ---------------------------------------------------------------------------
template <int D, bool BF16, int CW>
struct ChainSmem {
  using Gm = Geo<D, BF16>;
  static constexpr size_t KQ = Gm::KQ_BYTES;
  static constexpr size_t TP = 8 * Gm::KSC * kTileBytes;
  static constexpr size_t VC = CW * 4 * Pk<BF16>::VC_BYTES;
  static constexpr size_t GATES = Gm::GATE_BYTES;
  static constexpr size_t BUF = KQ + TP + VC + GATES;
  static constexpr int UNITS = static_cast<int>(BUF / 16);           // 16-byte units per buffer
  static constexpr int NBUF = 2 * BUF <= 150 * 1024 ? 2 : 1;
  static constexpr size_t BYTES = NBUF * BUF;
};

template <int D, bool BF16, int CW>
__global__ __launch_bounds__(CW * 64, 1) void chain_kernel(PrefillArgs A, PrefillLayout Lay) {
  using P = Pk<BF16>;
  using Gm = Geo<D, BF16>;
  using Sm = ChainSmem<D, BF16, CW>;
  using Ch = Chain<BF16>;
  using E = typename P::E;
  using Bop = typename Ch::Bop;
  constexpr int KSD = Gm::KSD, KSC = Gm::KSC, NT = Gm::NT;
  constexpr int TPS = P::SK / 16;                 // accumulator tiles per packed super-step
  constexpr int U_KQ = static_cast<int>(Sm::KQ / 16);
  constexpr int U_TP = U_KQ + static_cast<int>(Sm::TP / 16);
  constexpr int U_VC = U_TP + static_cast<int>(Sm::VC / 16);
  __shared__ __attribute__((aligned(1024))) char lds0[Sm::BUF];
  __shared__ __attribute__((aligned(1024))) char lds1[Sm::NBUF == 2 ? Sm::BUF : 16];

  const int s = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dvt = blockIdx.z * CW + wave;        // this wave's 16 rows of d_v
  const int32_t* se = ws_ptr<int32_t>(A.workspace, Lay.seq_tab) + 8 * s;
  if (!(se[SQ_FLAGS] & SQF_VALID)) return;
  const bool init = (se[SQ_FLAGS] & SQF_INIT) != 0;
  const int first = se[SQ_FIRST], nc = se[SQ_NCHUNK], slot = se[SQ_SLOT];
  const int seq_start = se[SQ_START], len = se[SQ_LEN];
  const uint32_t pos0 = static_cast<uint32_t>(se[SQ_POS0]);
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk, kh = h / G;
  const int g = lane >> 4, col = lane & 15;

  // ---- S^T slice in accumulators: tile i holds S^T[16i + 4g + e][16 dvt + col] ----
  float* Sglob = A.state + (static_cast<size_t>(slot) * Hv + h) * D * D + static_cast<size_t>(16 * dvt + col) * D;
  f32x4_t st[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if (init) {
      const float4 v = *reinterpret_cast<const float4*>(Sglob + 16 * i + 4 * g);
      st[i] = f32x4_t{v.x, v.y, v.z, v.w};
    } else {
      st[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Staging of one chunk into one LDS buffer with direct global->LDS loads:
  // the packed K/Q/K^T block of the k-head, the T/P tiles, this workgroup's V
  // tiles and the gate factors of the head.  The two buffers are distinct LDS
  // arrays, so loads landing in one never make the compiler wait before
  // reading the other.
  const char* wsb = static_cast<const char*>(A.workspace);
  // Every 1 KB block of the buffer lies in one segment (the segment sizes are
  // multiples of 1 KB), so the source base is wave-uniform and each lane adds
  // its 16-byte offset.
  static_assert(Sm::KQ % 1024 == 0 && Sm::TP % 1024 == 0 && Sm::VC % 512 == 0, "segment alignment");
  auto stage = [&](int chunk, char* base) {
    const char* kq = wsb + Lay.kq + (static_cast<size_t>(chunk) * Hk + kh) * Gm::KQ_BYTES;
    const char* hb = wsb + Lay.head + (static_cast<size_t>(chunk) * Hv + h) * Gm::HEAD_BYTES;
    const char* vcb = hb + Gm::VC_OFF + static_cast<size_t>(blockIdx.z) * CW * 4 * P::VC_BYTES;
    constexpr int NKQ = static_cast<int>(Sm::KQ / 1024), NTP = static_cast<int>(Sm::TP / 1024);
    auto dma = [&](const char* src, char* dst, int lim) {
      if (lane * 16 < lim)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4*>(src) + lane,
                                         (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
    };
    for (int b = wave; b < NKQ; b += CW) dma(kq + b * 1024, base + b * 1024, 1024);
    for (int b = wave; b < NTP; b += CW) dma(hb + b * 1024, base + Sm::KQ + b * 1024, 1024);
    for (int b = wave; b * 1024 < static_cast<int>(Sm::VC); b += CW)
      dma(vcb + b * 1024, base + Sm::KQ + Sm::TP + b * 1024, static_cast<int>(Sm::VC) - b * 1024);
    if (wave == CW - 1) dma(hb + Gm::GATE_OFF, base + Sm::KQ + Sm::TP + Sm::VC, static_cast<int>(Sm::GATES));
  };
  auto wait_stage = [&]() {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads have landed
    lds_barrier();                  // ... and everyone else's
  };

  // One chunk step from LDS buffer buf; O returned in registers.
  auto compute = [&](const char* base, f32x4_t (&O)[4]) {
    const uint4* kq = reinterpret_cast<const uint4*>(base);
    const uint4* tp = reinterpret_cast<const uint4*>(base + Sm::KQ);
    const E* vc = reinterpret_cast<const E*>(base + Sm::KQ + Sm::TP) + wave * 4 * 256;
    const float* gt = reinterpret_cast<const float*>(base + Sm::KQ + Sm::TP + Sm::VC);
    auto tileA = [&](const uint4* arr, int t) { return arr[t * 64 + lane]; };

    // B operands of S^T (d_k in packed order)
    Bop bS[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      const int i0 = ks * TPS;
      bS[ks] = Ch::bop(st[i0], (TPS == 2 && i0 + 1 < NT) ? st[(i0 + 1) % NT] : f32x4_t{0.f, 0.f, 0.f, 0.f});
    }
    // X = K S^T and Y = Q S^T for the 4 token tiles
    f32x4_t X[4], Y[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      X[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      Y[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        X[mt] = Ch::step(tileA(kq + Gm::KA * 64, mt * KSD + ks), bS[ks], X[mt]);
        Y[mt] = Ch::step(tileA(kq + Gm::QA * 64, mt * KSD + ks), bS[ks], Y[mt]);
      }
    }
    // R = beta V - (beta e^G) X for this lane's tokens 16 mt + 4 g + i
    f32x4_t Rt[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 c1 = *reinterpret_cast<const float4*>(gt + kC + 16 * mt + 4 * g);
      float vv[4];
      if constexpr (BF16) {
        const uint2 r2 = *reinterpret_cast<const uint2*>(vc + mt * 256 + lane * 4);
        vv[0] = __uint_as_float(r2.x << 16); vv[1] = __uint_as_float(r2.x & 0xffff0000u);
        vv[2] = __uint_as_float(r2.y << 16); vv[3] = __uint_as_float(r2.y & 0xffff0000u);
      } else {
        const float4 r4 = *reinterpret_cast<const float4*>(vc + mt * 256 + lane * 4);
        vv[0] = r4.x; vv[1] = r4.y; vv[2] = r4.z; vv[3] = r4.w;
      }
      Rt[mt][0] = fmaf(-c1.x, X[mt][0], vv[0]);
      Rt[mt][1] = fmaf(-c1.y, X[mt][1], vv[1]);
      Rt[mt][2] = fmaf(-c1.z, X[mt][2], vv[2]);
      Rt[mt][3] = fmaf(-c1.w, X[mt][3], vv[3]);
    }
    // U = T R (T lower triangular: token tile mt needs j < 16 (mt + 1))
    Bop bR[KSC];
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) bR[ks] = Ch::bop(Rt[ks * TPS], Rt[(ks * TPS + 1) % 4]);
    f32x4_t U[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      U[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks)
        if (ks * P::SK < 16 * (mt + 1)) U[mt] = Ch::step(tileA(tp + Gm::TA * 64, mt * KSC + ks), bR[ks], U[mt]);
    }
    // O = diag(e^G) Y + P U;  Ut = diag(e^{G_last - G}) U
    f32x4_t Ut[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 dc = *reinterpret_cast<const float4*>(gt + 2 * kC + 16 * mt + 4 * g);
      Ut[mt] = U[mt] * f32x4_t{dc.x, dc.y, dc.z, dc.w};
    }
    Bop bU[KSC], bUt[KSC];
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      bU[ks] = Ch::bop(U[ks * TPS], U[(ks * TPS + 1) % 4]);
      bUt[ks] = Ch::bop(Ut[ks * TPS], Ut[(ks * TPS + 1) % 4]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const float4 eg = *reinterpret_cast<const float4*>(gt + 16 * mt + 4 * g);
      f32x4_t o = Y[mt] * f32x4_t{eg.x, eg.y, eg.z, eg.w};
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks)
        if (ks * P::SK < 16 * (mt + 1)) o = Ch::step(tileA(tp + Gm::PA * 64, mt * KSC + ks), bU[ks], o);
      O[mt] = o;
    }
    // S^T <- e^{G_last} S^T + K^T Ut
    const float eGl = gt[3 * kC];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      f32x4_t acc = st[i] * eGl;
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) acc = Ch::step(tileA(kq + Gm::KTA * 64, i * KSC + ks), bUt[ks], acc);
      st[i] = acc;
    }
  };

  // O of chunk ci (tokens seq_start + 64 ci + 16 mt + 4 g + i, column 16 dvt + col)
  const size_t rowstride = static_cast<size_t>(Hv) * D;
  auto store_o = [&](int ci, const f32x4_t (&O)[4]) {
    const int clen = min(kC, len - kC * ci);
    E* ob = static_cast<E*>(A.o) + (static_cast<size_t>(seq_start + kC * ci + 4 * g)) * rowstride + h * D + 16 * dvt + col;
    if (clen == kC) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) ob[(16 * mt + i) * rowstride] = to_e<BF16>(O[mt][i]);
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * mt + 4 * g + i < clen) ob[(16 * mt + i) * rowstride] = to_e<BF16>(O[mt][i]);
    }
  };

  if (nc > 0) {
    f32x4_t O[4];
    stage(first, lds0);
    wait_stage();
    for (int ci = 0; ci < nc; ci += 2) {
      if (Sm::NBUF == 2) {
        if (ci + 1 < nc) stage(first + ci + 1, lds1);
        if (ci > 0) store_o(ci - 1, O);
        compute(lds0, O);
        wait_stage();
        if (ci + 1 < nc) {
          if (ci + 2 < nc) stage(first + ci + 2, lds0);
          store_o(ci, O);
          compute(lds1, O);
          wait_stage();
        }
      } else {
        if (ci > 0) store_o(ci - 1, O);
        compute(lds0, O);
        if (ci + 1 < nc) {
          lds_barrier();
          stage(first + ci + 1, lds0);
          wait_stage();
          store_o(ci, O);
          compute(lds0, O);
          if (ci + 2 < nc) {
            lds_barrier();
            stage(first + ci + 2, lds0);
            wait_stage();
          }
        }
      }
    }
    store_o(nc - 1, O);
  }

  // ---- final state back to the slot ----
#pragma unroll
  for (int i = 0; i < NT; ++i)
    *reinterpret_cast<float4*>(Sglob + 16 * i + 4 * g) = make_float4(st[i][0], st[i][1], st[i][2], st[i][3]);

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
      for (int cc = tid; cc < 2 * D; cc += CW * 64) put(cc < D ? kh * D + cc : Hk * D + kh * D + (cc - D));
    if (lane < 16) put(2 * Hk * D + h * D + 16 * dvt + lane);
    if (h == 0 && blockIdx.z == 0 && tid == 0) A.conv_pos[slot] = static_cast<int32_t>(pos_end << kPosShift);
  }
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------
template <int D, bool BF16>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  constexpr int CW = Geo<D, BF16>::NT < 2 ? Geo<D, BF16>::NT : 2;
  const PrefillLayout L = layout_t<D, BF16>(a.Hk, a.Hv, a.max_chunks, a.n_seqs);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, a, L);
  int e = static_cast<int>(hipGetLastError());
  if (e) return e;
  const size_t smem = ChunkSmem<D, BF16>::BYTES;
  e = static_cast<int>(hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_kernel<D, BF16>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem)));
  if (e) return e;
  if (a.max_chunks > 0) {
    hipLaunchKernelGGL((chunk_kernel<D, BF16>), dim3(a.max_chunks, a.Hk), dim3(kChunkThreads), smem, st, a, L);
    e = static_cast<int>(hipGetLastError());
    if (e) return e;
  }
  hipLaunchKernelGGL((chain_kernel<D, BF16, CW>), dim3(a.n_seqs, a.Hv, Geo<D, BF16>::NT / CW), dim3(CW * 64), 0,
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
