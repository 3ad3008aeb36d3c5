// Chunked (WY / UT-transform) prefill of the gated delta rule on gfx950.
//
// Inside a chunk of n <= 64 tokens of one sequence, with cumulative log-gates
// G_r = sum_{j<=r} g_j and the state S at the chunk start (d_v x d_k):
//   L_rj = beta_r e^{G_r - G_j} (k_r . k_j)   for r > j (0 otherwise)
//   T    = (I + L)^{-1}                                      (unit lower triangular)
//   W    = T diag(beta e^G) K,   U' = T diag(beta) V        (chunk-local)
//   U    = U' - W S^T                                        (the corrected writes u_r)
//   O    = diag(e^G) Q S^T + P U,  P_rj = e^{G_r - G_j} (q_r . k_j) for j <= r
//   S   <- e^{G_last} S + U^T diag(e^{G_last - G}) K
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
//           cumulative sums, K K^T and K Q^T on MFMA, then per v-head P, the
//           inverse T, W and U'.  Everything the next kernel multiplies is
//           written pre-packed in MFMA operand order (below);
//   chain:  one wave per (sequence, v-head, 16 rows of d_v) walks the
//           sequence's chunks in order.  It keeps its 16 x d_k slice of the
//           state, transposed, in MFMA accumulators and never leaves
//           registers: every product's result feeds the next product as its
//           B operand directly (the contraction order inside an MFMA is a
//           free permutation, so the A operand is packed in the permuted
//           order that matches the accumulator layout).  Per chunk it does
//           only what depends on the state: U = U' - W S^T, Q S^T, P U and
//           the state update.  The waves of a workgroup share the chunk's
//           packed operands, staged into LDS with direct global->LDS loads
//           one chunk ahead.
//
// Packed operand tiles.  A 16 x SK sub-matrix (rows r, contraction index k;
// SK = 32 for the bf16 MFMA 16x16x32, 16 for four fp32 MFMA 16x16x4) is
// stored as 64 lanes x 16 bytes.  Lane (g = k%16 / 4) * 16 + r holds, in
// element e = (k / 16) * 4 + k % 4, the value at (r, k).  A 16x16
// accumulator tile holds rows 4g..4g+3 of column l%16 in lane l, so the
// accumulators of tiles (2s, 2s+1) (bf16) or tile s (fp32) form exactly the
// B operand that pairs with packed tile column s -- and, read the other way,
// the packed A tile of the transposed product.
#include <mutex>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

#ifndef GDN_CHAIN_SCHED
#define GDN_CHAIN_SCHED 1
#endif

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
  static constexpr int TPS = P::SK / 16;               // accumulator tiles per packed super-step
  // per (chunk, k-head): Q as A (rows token, k = d), 4 x KSD tiles
  static constexpr size_t KQ_BYTES = 4 * KSD * kTileBytes;
  // per (chunk, v-head), in this order:
  static constexpr int WA = 0;                 // -W as A (rows token, k = d):                     4 x KSD
  static constexpr int KDA = 4 * KSD;          // (diag(e^{G_last - G}) K)^T as A (rows d, k = tok): NT x KSC
  static constexpr int PA = KDA + NT * KSC;    // P as A (rows r, k = j):                           4 x KSC
  static constexpr int HT_TILES = PA + 4 * KSC;
  static constexpr size_t VW_OFF = HT_TILES * kTileBytes;           // U', accumulator layout [NT][4]
  static constexpr size_t GATE_OFF = VW_OFF + NT * 4 * P::VC_BYTES;  // e^G (64 floats), e^{G_last} (64 copies)
  static constexpr size_t GATE_BYTES = 2 * kC * 4;
  static constexpr size_t VB_OFF = GATE_OFF + GATE_BYTES;            // V, accumulator layout [NT][4] (chunk kernel)
  static constexpr size_t HEAD_BYTES = VB_OFF + NT * 4 * P::VC_BYTES;
};

// Sequence s needs ceil(len_s / C) chunks, and the sum of those is at most
// floor((n_tokens + (C - 1) n_seqs) / C).
int prefill_max_chunks(int n_tokens, int n_seqs) {
  return static_cast<int>((static_cast<int64_t>(n_tokens) + static_cast<int64_t>(kC - 1) * n_seqs) / kC);
}

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
  L.chunk_tab = take(mc * 8 * 4);
  L.seq_tab = take(static_cast<size_t>(S) * 8 * 4);
  L.ready = take(mc * Hk * 4);
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
// SQ_CKPT0: index of the sequence's first state checkpoint.
enum { SQ_FIRST = 0, SQ_NCHUNK, SQ_POS0, SQ_FLAGS, SQ_SLOT, SQ_START, SQ_LEN, SQ_CKPT0 };
enum { SQF_VALID = 1, SQF_INIT = 2 };
// Chunk table entry (int32 x 8, one per chunk up to the bound): everything a
// chunk workgroup needs in one 32-byte read.  CT_LEN is 0 past the last chunk.
enum { CT_T0 = 0, CT_LEN, CT_SEQ_START, CT_SLOT, CT_FLAGS, CT_POS0, CT_PAD0, CT_PAD1 };

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
  __shared__ int s_total;
  if (threadIdx.x == 0) {
    const int S = A.n_seqs;
    bool ok = A.cu_seqlens[0] == 0 && A.cu_seqlens[S] == A.n_tokens;
    int bad_code = ok ? 0 : GDN_DEV_BAD_SEQLENS;
    int total = 0, n_ckpt = 0;
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
      e[SQ_POS0] = (init && A.W > 0 && ok) ? static_cast<int32_t>(static_cast<uint32_t>(A.conv_pos[slot * kPosStride]) >> kPosShift) : 0;
      e[SQ_FLAGS] = SQF_VALID | (init ? SQF_INIT : 0);
      e[SQ_SLOT] = slot;
      e[SQ_START] = st;
      e[SQ_LEN] = len;
      e[SQ_CKPT0] = n_ckpt;
      total += nc;
      if (A.ckpt_every > 0 && len > 0) n_ckpt += len / A.ckpt_every;
    }
    if (!ok) {
      report_error(A.dev_err, bad_code);
      for (int s = 0; s < S; ++s) stab[8 * s + SQ_FLAGS] = 0;
      total = 0;
    }
    if (total > A.max_chunks) total = 0;  // cannot happen for a valid partition
    s_total = total;
  }
  // every (chunk, k-head) starts unpublished
  int32_t* ready = ws_ptr<int32_t>(A.workspace, L.ready);
  for (int i = threadIdx.x; i < A.max_chunks * A.Hk; i += blockDim.x) ready[i] = 0;
  __syncthreads();
  const int total = s_total;
  for (int c = threadIdx.x; c < A.max_chunks; c += blockDim.x) {
    int32_t* e = ctab + 8 * c;
    if (c >= total) {
      for (int k = 0; k < 8; ++k) e[k] = 0;  // no chunk: CT_LEN 0
      continue;
    }
    int lo = 0, hi = A.n_seqs - 1;  // last s with first <= c holds c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (stab[8 * mid + SQ_FIRST] <= c) lo = mid; else hi = mid - 1;
    }
    const int32_t* q = stab + 8 * lo;
    const int i = c - q[SQ_FIRST];
    e[CT_T0] = q[SQ_START] + i * kC;
    e[CT_LEN] = min(kC, q[SQ_LEN] - i * kC);
    e[CT_SEQ_START] = q[SQ_START];
    e[CT_SLOT] = q[SQ_SLOT];
    e[CT_FLAGS] = q[SQ_FLAGS];
    e[CT_POS0] = q[SQ_POS0];
    e[CT_PAD0] = 0;
    e[CT_PAD1] = 0;
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
__device__ __forceinline__ void invert_unit_lower64(float* Lt, float* tmp, int lane) {
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
// chunk: front end, gates, K K^T / K Q^T, then per v-head P, T, W and U'
// (8 waves)
// ---------------------------------------------------------------------------
// 12 waves: the 640 conv items at G = 3, d = 128 spread evenly over the 4 SIMDs
constexpr int kChunkThreads = 768;
constexpr int kChunkWaves = kChunkThreads / 64;

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// LDS of the chunk kernel, by lifetime:
//   R0: conv outputs of q | k (fp32), then L -> T and inverse scratch of NH heads
//   R1: k (hi, lo for bf16) and q as A tiles, then T diag(beta e^G), T diag(beta) of NH heads
//   KT: K^T as A tiles;  AM: K K^T;  MISC: per-token gate tables and norm factors
template <int D, bool BF16>
struct ChunkSmem {
  using Gm = Geo<D, BF16>;
  static constexpr int NH = BF16 ? 3 : 1;            // v-heads per inverse group
  static constexpr int QK_LD = 2 * D + 4;            // rows 16-byte aligned
  static constexpr int PK_Q = BF16 ? 2 : 1;          // index of the q tiles in R1
  static constexpr size_t LT1 = static_cast<size_t>(kC) * kLd * 4;
  static constexpr size_t SCR1 = 32 * 33 * 4;
  static constexpr size_t R0 = cmax(static_cast<size_t>(kC) * QK_LD * 4, NH * (LT1 + SCR1));
  static constexpr size_t TT1 = 2 * 4 * Gm::KSC * kTileBytes;
  static constexpr size_t R1 = cmax((PK_Q + 1) * 4 * Gm::KSD * kTileBytes, NH * TT1);
  static constexpr size_t KT = static_cast<size_t>(Gm::NT) * Gm::KSC * kTileBytes;
  static constexpr size_t AM = LT1;
  static constexpr size_t MISC = static_cast<size_t>(4 * kMaxGroup * kC + 2 * kC) * 4;
  static constexpr size_t BYTES = R0 + R1 + KT + AM + MISC;
};

// The chunk tile list of the P products: (row tile ti, packed column ks) with
// ks * SK <= 16 ti + 15, i.e. the tiles of a lower-triangular 64x64 matrix
// that are not identically zero.
template <bool BF16>
struct TriTiles {
  static constexpr int SK = Pk<BF16>::SK;
  static constexpr int count() {
    int n = 0;
    for (int ti = 0; ti < 4; ++ti) n += (16 * ti + 15) / SK + 1;
    return n;
  }
  __device__ static void at(int t, int& ti, int& ks) {
    ti = 0;
    while (t > (16 * ti + 15) / SK) { t -= (16 * ti + 15) / SK + 1; ++ti; }
    ks = t;
  }
};

// KW: conv width, 4 or 0 (inputs are q | k | v directly); a compile-time
// constant so the unrolled per-token conv code has no branches.
template <int D, bool BF16, int KW>
__global__ __launch_bounds__(kChunkThreads) void chunk_kernel(PrefillArgs A, PrefillLayout Lay) {
  using P = Pk<BF16>;
  using Gm = Geo<D, BF16>;
  using Sm = ChunkSmem<D, BF16>;
  using Ch = Chain<BF16>;
  using Bop = typename Ch::Bop;
  using E = typename P::E;
  constexpr int VE = 4;                          // channels per conv item (one 8- or 16-byte load per row)
  using RawT = typename std::conditional<BF16, uint2, uint4>::type;
  constexpr int KSD = Gm::KSD, KSC = Gm::KSC, NT = Gm::NT, TPS = Gm::TPS, SK = P::SK, EPL = P::EPL;
  constexpr int NH = Sm::NH, QK_LD = Sm::QK_LD;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  char* sb = reinterpret_cast<char*>(smem);
  float* qk = smem;                                        // [64][QK_LD] conv outputs of q | k
  float* Lt = smem;                                        // NH x [64][65]: L -> T
  float* tmpw = smem + NH * kC * kLd;                      // NH x [32][33] inverse scratch
  uint4* pk = reinterpret_cast<uint4*>(sb + Sm::R0);       // k (hi, lo) and q as A tiles
  uint4* tt = pk;                                          // NH x 2 x [4 x KSC] T tiles
  uint4* kt = reinterpret_cast<uint4*>(sb + Sm::R0 + Sm::R1);  // K^T as A: NT x KSC tiles
  float* Am = reinterpret_cast<float*>(sb + Sm::R0 + Sm::R1 + Sm::KT);  // [64][65] K K^T
  float* gcum = Am + kC * kLd;                             // [8][64] G
  float* bet = gcum + kMaxGroup * kC;                      // [8][64] beta
  float* dkf = bet + kMaxGroup * kC;                       // [8][64] e^{G_last - G}
  float* bge = dkf + kMaxGroup * kC;                       // [8][64] beta e^G
  float* inv = bge + kMaxGroup * kC;                       // [2][64] q and k norm factors

  // grid (k-heads, chunks): workgroups are dispatched chunk by chunk, the
  // order in which the chain kernel consumes them
  const int chunk = A.seg_lo + blockIdx.y;
  const int kh = blockIdx.x;
  // one read of the chunk's table entry (no chain of dependent reads)
  const int32_t* ce = ws_ptr<int32_t>(A.workspace, Lay.chunk_tab) + 8 * chunk;
  const int t0 = ce[CT_T0], len = ce[CT_LEN];
  if (len <= 0) return;
  const bool init = (ce[CT_FLAGS] & SQF_INIT) != 0;
  const uint32_t pos0 = static_cast<uint32_t>(ce[CT_POS0]);
  const int slot = ce[CT_SLOT];
  const int seq_start = ce[CT_SEQ_START];
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk, C = A.C, R = A.R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const E* x = static_cast<const E*>(A.x);
  char* kqb = static_cast<char*>(A.workspace) + Lay.kq + (static_cast<size_t>(chunk) * Hk + kh) * Gm::KQ_BYTES;
  auto headb = [&](int h) {
    return static_cast<char*>(A.workspace) + Lay.head + (static_cast<size_t>(chunk) * Hv + h) * Gm::HEAD_BYTES;
  };
  auto xchan = [&](int cc) {
    return cc < D ? kh * D + cc : (cc < 2 * D ? Hk * D + kh * D + (cc - D) : 2 * Hk * D + kh * G * D + (cc - 2 * D));
  };

  // gate inputs of the v-head whose gates this wave computes (the first G
  // waves, one head each: q|k waves, whose conv items end before the v
  // items, which also store V), loaded before the conv so they arrive under
  // it; they stay raw until the gates are computed, so nothing waits for them here
  static_assert(kMaxGroup <= kChunkWaves, "one gate head per wave");
  const int ghi = wave;
  E a_raw{}, b_raw{};
  if (ghi < G && lane < len) {
    const size_t i = static_cast<size_t>(t0 + lane) * Hv + kh * G + ghi;
    a_raw = static_cast<const E*>(A.a)[i];
    b_raw = static_cast<const E*>(A.b)[i];
  }

  // ---- conv + SiLU: item = (VE channels, 16 tokens), the 19-row window in registers.
  // q|k items first, then v items; each wave takes a contiguous run of items
  // of one kind. ----
  {
    const int nvq = 2 * D / VE, nvv = G * D / VE;
    const int n_qk = 4 * nvq, n_items = 4 * (nvq + nvv);
    // q|k items on the first wq waves, v items on the rest, in proportion, so
    // that no wave holds both kinds (a wave would run both code paths)
    const int wq = max(1, min(kChunkWaves - 1, (2 * kChunkWaves * n_qk + n_items) / (2 * n_items)));
    const bool qk_wave = wave < wq;
    const int ipw = qk_wave ? (n_qk + wq - 1) / wq : (n_items - n_qk + kChunkWaves - wq - 1) / (kChunkWaves - wq);
    const int item0 = qk_wave ? wave * ipw : n_qk + (wave - wq) * ipw;
    const int item_end = qk_wave ? n_qk : n_items;
    auto conv_item = [&](int jj) __attribute__((always_inline)) {
      const int item = item0 + jj;
      if (item >= item_end) return;
      int q, vec;
      if (item < 4 * nvq) {
        q = item / nvq;
        vec = item - q * nvq;
      } else {
        const int i2 = item - 4 * nvq;
        q = i2 / nvv;
        vec = nvq + (i2 - q * nvv);
      }
      const int cc0 = vec * VE;
      const int c0 = xchan(cc0);
      const int tq = 16 * q;                        // first token of this quarter
      // raw rows: tokens t0+tq-3 .. t0+tq+15 (row i <-> token t0+tq-3+i),
      // clamped into the sequence and the chunk so every load is valid; an
      // interior quarter needs no clamping, so its row addresses are one
      // stride apart
      RawT raw[19];
      const int tfirst = t0 + tq - 3;
      if (tfirst >= seq_start && tq + 16 <= len) {
        const E* xr = x + static_cast<size_t>(tfirst) * C + c0;
#pragma unroll
        for (int i = 0; i < 19; ++i) raw[i] = *reinterpret_cast<const RawT*>(xr + static_cast<size_t>(i) * C);
      } else {
#pragma unroll
        for (int i = 0; i < 19; ++i) {
          const int t = min(max(tfirst + i, seq_start), t0 + len - 1);
          raw[i] = *reinterpret_cast<const RawT*>(x + static_cast<size_t>(t) * C + c0);
        }
      }
      // conv weights times -log2(e): the conv then yields -log2(e) y, the
      // argument the SiLU's exp2 takes
      float w[VE][4];
      if constexpr (KW == 4) {
#pragma unroll
        for (int v = 0; v < VE; ++v) {
          const float4 w4 = *reinterpret_cast<const float4*>(A.conv_w + (c0 + v) * 4);
          w[v][0] = kNegLog2e * w4.x; w[v][1] = kNegLog2e * w4.y;
          w[v][2] = kNegLog2e * w4.z; w[v][3] = kNegLog2e * w4.w;
        }
      }
      auto elem = [&](const RawT& r, int v) -> float {
        if constexpr (BF16) {
          const uint32_t wv = v < 2 ? r.x : r.y;
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
      E* vcb = reinterpret_cast<E*>(headb(kh * G + hv) + Gm::VB_OFF);
      // tokens past the end of a ragged chunk give zero rows
      auto run = [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {              // 4 groups of 4 tokens
          float y[VE][4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;                 // token within the quarter
#pragma unroll
            for (int v = 0; v < VE; ++v) {
              const float xin = elem(raw[3 + r], v);
              float yy;
              if constexpr (KW == 4) {
                float acc = w[v][0] * hist[v][0];
                acc = fmaf(w[v][1], hist[v][1], acc);
                acc = fmaf(w[v][2], hist[v][2], acc);
                acc = fmaf(w[v][3], xin, acc);
                yy = silu_of_scaled(acc);
                hist[v][0] = hist[v][1]; hist[v][1] = hist[v][2]; hist[v][2] = xin;
              } else {
                yy = xin;
              }
              y[v][i] = (FULL || tq + r < len) ? yy : 0.f;
            }
          }
          if (!is_v) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float* dst = qk + (tq + 4 * g4 + i) * QK_LD + cc0;
#pragma unroll
              for (int v = 0; v < VE; v += 4)
                *reinterpret_cast<float4*>(dst + v) = make_float4(y[v][i], y[v + 1][i], y[v + 2][i], y[v + 3][i]);
            }
          } else {
            // accumulator layout: tile (dv/16, quarter q), lane g4*16 + dv%16,
            // elements i.  The VE channels of an item sit side by side in one
            // row of a tile (dv0 is a multiple of VE), so bf16 goes out as two
            // 16-byte stores and four lanes fill a 128-byte line.
            E* dst = vcb + ((dv0 >> 4) * 4 + q) * 256 + (g4 * 16 + (dv0 & 15)) * 4;
            static_assert(VE == 4, "four channels per item");
            if constexpr (BF16) {
#pragma unroll
              for (int v = 0; v < VE; v += 2)
                *reinterpret_cast<uint4*>(dst + 4 * v) =
                    make_uint4(pack2_bf16(y[v][0], y[v][1]), pack2_bf16(y[v][2], y[v][3]),
                               pack2_bf16(y[v + 1][0], y[v + 1][1]), pack2_bf16(y[v + 1][2], y[v + 1][3]));
            } else {
#pragma unroll
              for (int v = 0; v < VE; ++v)
                *reinterpret_cast<float4*>(dst + 4 * v) = make_float4(y[v][0], y[v][1], y[v][2], y[v][3]);
            }
          }
        }
      };
      if (tq + 16 <= len) run(std::true_type{});
      else run(std::false_type{});
    };
    // the first item outside the loop: its loads go out right behind the
    // gate inputs, with no wait between
    if (lane < ipw) conv_item(lane);
    for (int jj = lane + 64; jj < ipw; jj += 64) conv_item(jj);
  }

  // ---- gates: one wave per v-head (the first waves), lane = token, fixed-order inclusive scan ----
  if (ghi < G) {
    const int hi = ghi, h = kh * G + hi;
    float g = 0.f, bb = 0.f;
    // the opaque copy keeps the compiler from converting (and so waiting
    // for) the raw inputs before the conv
    asm volatile("" : "+v"(a_raw), "+v"(b_raw));
    if (lane < len) {
      float a_in, b_in;
      if constexpr (BF16) {
        a_in = bf16_bits_to_f32(a_raw);
        b_in = bf16_bits_to_f32(b_raw);
      } else {
        a_in = a_raw;
        b_in = b_raw;
      }
      g = -softplus_f(a_in);
      bb = sigmoid_f(b_in);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float up = __shfl_up(g, off, 64);
      if (lane >= off) g += up;
    }
    const float glast = __shfl(g, 63, 64);
    const float eg = __expf(g);
    gcum[hi * kC + lane] = g;
    bet[hi * kC + lane] = bb;
    dkf[hi * kC + lane] = __expf(glast - g);
    bge[hi * kC + lane] = bb * eg;
    float* gw = reinterpret_cast<float*>(headb(h) + Gm::GATE_OFF);
    store_wt(gw, 4 * lane, eg);
    store_wt(gw, 4 * (kC + lane), __expf(glast));
  }

  __syncthreads();

  // ---- L2 norm factors of q and k per token: 8 lanes per token, fixed order ----
  {
    const bool norm = (A.flags & GDN_FLAG_L2NORM_QK) != 0;
    constexpr int PER = D / 8;
    const int r = (wave & 7) * 8 + (lane >> 3), part = lane & 7;  // waves 0-7: 8 tokens each
    const float* qr = qk + r * QK_LD + part * PER;
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float a = qr[e], b = qr[D + e];
      sq = fmaf(a, a, sq);
      sk = fmaf(b, b, sk);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
      sq += __shfl_xor(sq, off, 64);
      sk += __shfl_xor(sk, off, 64);
    }
    if (part == 0 && wave < 8) {
      inv[r] = norm ? A.q_scale * (1.0f / sqrtf(sq + A.l2_eps)) : A.q_scale;
      inv[kC + r] = norm ? 1.0f / sqrtf(sk + A.l2_eps) : 1.0f;
    }
  }
  __syncthreads();
  auto qn = [&](int r, int d) { return qk[r * QK_LD + d] * inv[r]; };
  auto kn = [&](int r, int d) { return qk[r * QK_LD + D + d] * inv[kC + r]; };
  auto pack = [&](const float (&v)[EPL]) { return pack_lane<BF16>([&](int e) { return v[e]; }); };

  // ---- packing: K (hi, lo) and Q as A tiles (rows token, k = d) into LDS, Q also
  // to the workspace; K^T as A (rows d, k = token) into LDS; per v-head
  // (diag(e^{G_last - G}) K)^T to the workspace ----
  for (int u = tid; u < 4 * KSD * 64; u += kChunkThreads) {
    const int tile = u >> 6, ln = u & 63;
    const int mt = tile / KSD, ks = tile % KSD;
    const int row = 16 * mt + (ln & 15), g = ln >> 4;
    float kv[EPL], qv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int k = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
      kv[e] = k < D ? kn(row, k) : 0.f;
      qv[e] = k < D ? qn(row, k) : 0.f;
    }
    const uint4 qw = pack(qv);
    store_wt(kqb, 16 * (tile * 64 + ln), qw);
    pk[(Sm::PK_Q * 4 * KSD + tile) * 64 + ln] = qw;
    pk[tile * 64 + ln] = pack(kv);
    if constexpr (BF16) {
      float lo[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) lo[e] = kv[e] - bf16_bits_to_f32(f32_to_bf16_bits(kv[e]));
      pk[(4 * KSD + tile) * 64 + ln] = pack(lo);
    }
  }
  for (int u = tid; u < NT * KSC * 64; u += kChunkThreads) {
    const int tile = u >> 6, ln = u & 63;
    const int dt = tile / KSC, ks = tile % KSC;
    const int dk = 16 * dt + (ln & 15), g = ln >> 4;
    float kv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) kv[e] = kn(ks * SK + (e >> 2) * 16 + 4 * g + (e & 3), dk);
    kt[tile * 64 + ln] = pack(kv);
    for (int hi = 0; hi < G; ++hi) {
      const float* dk_h = dkf + hi * kC;
      float dv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) dv[e] = kv[e] * dk_h[ks * SK + (e >> 2) * 16 + 4 * g + (e & 3)];
      store_wt(headb(kh * G + hi), (Gm::KDA + tile) * kTileBytes + 16 * ln, pack(dv));
    }
  }
  __syncthreads();

  // ---- K K^T (lower 16x16 tiles) into LDS; K Q^T read as packed P tiles of
  // every v-head (workspace).  With a single inverse group the P tasks run on
  // the waves the inverse leaves idle. ----
  constexpr int NPT = TriTiles<BF16>::count();
  const uint4* kh_t = pk;
  const uint4* kl_t = pk + 4 * KSD * 64;
  const uint4* q_t = pk + Sm::PK_Q * 4 * KSD * 64;
  auto p_task = [&](int pt) {
    int ti, ks;
    TriTiles<BF16>::at(pt, ti, ks);
    // (K Q^T)[j][r] with j = 16 tj + 4g + i, r = 16 ti + (lane & 15): the
    // accumulator of tile (tj, ti) is packed P tile (ti, ks) element (tj%TPS)*4 + i
    f32x4_t acc[TPS];
#pragma unroll
    for (int u = 0; u < TPS; ++u) {
      const int tj = TPS * ks + u;
      acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (tj <= ti) {
#pragma unroll
        for (int kd = 0; kd < KSD; ++kd)
          acc[u] = Ch::step(kh_t[(tj * KSD + kd) * 64 + lane],
                            __builtin_bit_cast(Bop, q_t[(ti * KSD + kd) * 64 + lane]), acc[u]);
      }
    }
    const int r = 16 * ti + (lane & 15), g = lane >> 4;
    for (int hi = 0; hi < G; ++hi) {
      const float* gc = gcum + hi * kC;
      const float gr = gc[r];
      float pv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int j = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
        pv[e] = j <= r ? __expf(gr - gc[j]) * acc[e >> 2][e & 3] : 0.f;
      }
      store_wt(headb(kh * G + hi), (Gm::PA + ti * KSC + ks) * kTileBytes + 16 * lane, pack(pv));
    }
  };
  const bool p_later = G <= NH;
  {
    const int ntask = p_later ? 10 : 10 + NPT;
    for (int task = wave; task < ntask; task += kChunkWaves) {
      if (task < 10) {
        int t = task, ti = 0;
        while (t > ti) { t -= ti + 1; ++ti; }
        const int tj = t;
        // K K^T feeds the inverse: hi*hi + hi*lo + lo*hi for about fp32
        // accuracy, in three independent accumulators
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc1 = acc, acc2 = acc;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const uint4 ah = kh_t[(ti * KSD + ks) * 64 + lane];
          const Bop bh = __builtin_bit_cast(Bop, kh_t[(tj * KSD + ks) * 64 + lane]);
          acc = Ch::step(ah, bh, acc);
          if constexpr (BF16) {
            acc1 = Ch::step(ah, __builtin_bit_cast(Bop, kl_t[(tj * KSD + ks) * 64 + lane]), acc1);
            acc2 = Ch::step(kl_t[(ti * KSD + ks) * 64 + lane], bh, acc2);
          }
        }
        if constexpr (BF16) acc = acc + (acc1 + acc2);
        const int g = lane >> 4, j = 16 * tj + (lane & 15);
        if (G <= NH) {
          // one inverse group: L_rj = beta_r e^{G_r - G_j} (k_r . k_j), r > j, of every
          // v-head straight from the accumulator; the mirrored block above the
          // diagonal is zero
          for (int hi = 0; hi < G; ++hi) {
            const float* gc = gcum + hi * kC;
            const float gj = gc[j];
            float* Lh = Lt + hi * kC * kLd;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * ti + 4 * g + i;
              Lh[r * kLd + j] = j < r ? bet[hi * kC + r] * __expf(gc[r] - gj) * acc[i] : 0.f;
              if (ti != tj) Lh[(16 * tj + 4 * g + i) * kLd + 16 * ti + (lane & 15)] = 0.f;
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) Am[(ti * 16 + g * 4 + i) * kLd + j] = acc[i];
        }
      } else {
        p_task(task - 10);
      }
    }
  }
  __syncthreads();

  // ---- per group of NH v-heads: L, T = (I + L)^{-1}, then -W and U' ----
  for (int hg0 = 0; hg0 < G; hg0 += NH) {
    const int nh = min(NH, G - hg0);
    // U' = T diag(beta) V: task (head, dvt) makes the 4 token tiles of 16
    // columns.  The V tiles come from the workspace (L2): every wave
    // issues the loads of all its U' tasks before the inverse, so they are
    // in flight through the inverse, the T packing and the -W tasks.
    constexpr int MAXV = (NH * NT + kChunkWaves - 1) / kChunkWaves;
    const int nv = nh * NT;
    Bop vop[MAXV][KSC];
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
      const int t = min(wave + k * kChunkWaves, nv - 1);  // a clamped duplicate is loaded, never used
      const int i = t / NT, dvt = t % NT;
      const E* vb = reinterpret_cast<const E*>(headb(kh * G + hg0 + i) + Gm::VB_OFF) + dvt * 4 * 256 + lane * 4;
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        if constexpr (BF16) {
          const uint2 lo = *reinterpret_cast<const uint2*>(vb + (2 * ks) * 256);
          const uint2 hi = *reinterpret_cast<const uint2*>(vb + (2 * ks + 1) * 256);
          vop[k][ks] = __builtin_bit_cast(Bop, make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
          vop[k][ks] = __builtin_bit_cast(Bop, *reinterpret_cast<const uint4*>(vb + ks * 256));
        }
      }
    }
    if (G > NH) {  // several groups: L of this group from K K^T in LDS
      for (int e = tid; e < nh * kC * kC; e += kChunkThreads) {
        const int i = e / (kC * kC), r = (e / kC) % kC, j = e % kC;
        const float* gc = gcum + (hg0 + i) * kC;
        Lt[i * kC * kLd + r * kLd + j] = j < r ? bet[(hg0 + i) * kC + r] * __expf(gc[r] - gc[j]) * Am[r * kLd + j] : 0.f;
      }
      __syncthreads();
    }
    if (wave < nh) {
      invert_unit_lower64(Lt + wave * kC * kLd, tmpw + wave * 32 * 33, lane);
    } else if (p_later) {
      for (int pt = wave - nh; pt < NPT; pt += kChunkWaves - nh) p_task(pt);
    }
    __syncthreads();
    // T diag(beta e^G) (for W) and T diag(beta) (for U') as A tiles; the
    // identically zero tiles above the diagonal are never read
    for (int u = tid; u < nh * 2 * 4 * KSC * 64; u += kChunkThreads) {
      const int tile = (u >> 6) % (4 * KSC), which = (u >> 6) / (4 * KSC) % 2, i = (u >> 6) / (8 * KSC);
      const int ln = u & 63;
      const int mt = tile / KSC, ks = tile % KSC;
      if (ks * SK > 16 * mt + 15) continue;
      const int r = 16 * mt + (ln & 15), g = ln >> 4;
      const float* Ti = Lt + i * kC * kLd + r * kLd;
      const float* sc = (which == 0 ? bge : bet) + (hg0 + i) * kC;
      float tv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int j = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
        tv[e] = Ti[j] * sc[j];
      }
      tt[((i * 2 + which) * 4 * KSC + tile) * 64 + ln] = pack(tv);
    }
    __syncthreads();
    // -W = -(T diag(beta e^G)) K: W^T = K^T (T diag(beta e^G))^T, tile (dt, mt)
    // accumulators read as packed A tile (mt, ksd) of W (rows token, k = d)
    const int nw = nh * 4 * KSD;
    for (int task = wave; task < nw; task += kChunkWaves) {
      const int i = task / (4 * KSD), mt = (task / KSD) % 4, ksd = task % KSD;
      const int kmax = (16 * mt + 15) / SK;
      const uint4* tw = tt + (i * 2 + 0) * 4 * KSC * 64;
      f32x4_t acc[TPS];
#pragma unroll
      for (int u = 0; u < TPS; ++u) {
        const int dt = TPS * ksd + u;
        acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (dt < NT) {
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
            if (ks <= kmax)
              acc[u] = Ch::step(kt[(dt * KSC + ks) * 64 + lane],
                                __builtin_bit_cast(Bop, tw[(mt * KSC + ks) * 64 + lane]), acc[u]);
        }
      }
      float wv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) wv[e] = -acc[e >> 2][e & 3];
      store_wt(headb(kh * G + hg0 + i), (Gm::WA + mt * KSD + ksd) * kTileBytes + 16 * lane, pack(wv));
    }
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
      const int t = wave + k * kChunkWaves;
      if (t < nv) {
        const int i = t / NT, dvt = t % NT;
        const uint4* tb = tt + (i * 2 + 1) * 4 * KSC * 64;
        char* hbv = headb(kh * G + hg0 + i);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
            if (ks * SK <= 16 * mt + 15) acc = Ch::step(tb[(mt * KSC + ks) * 64 + lane], vop[k][ks], acc);
          if constexpr (BF16) {
            uint2 pkd;
            pkd.x = static_cast<uint32_t>(f32_to_bf16_bits(acc[0])) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
            pkd.y = static_cast<uint32_t>(f32_to_bf16_bits(acc[2])) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
            store_wt(hbv, Gm::VW_OFF + ((dvt * 4 + mt) * 256 + lane * 4) * sizeof(E), pkd);
          } else {
            store_wt(hbv, Gm::VW_OFF + ((dvt * 4 + mt) * 256 + lane * 4) * sizeof(E), make_float4(acc[0], acc[1], acc[2], acc[3]));
          }
        }
      }
    }
    __syncthreads();  // Lt and the T tiles are reused by the next group
  }

  // ---- publish (chunk, k-head) for a chain kernel running concurrently.
  // Everything the chain reads went out with write-through stores; once
  // every wave has seen its stores complete, the flag is set (itself a
  // write-through store) ----
  if (A.persistent) {
    wait_stores();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(ws_ptr<int32_t>(A.workspace, Lay.ready) + chunk * Hk + kh, 1, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// chain: sequential chunk loop, one wave per 16 rows of d_v
// ---------------------------------------------------------------------------
// s_sleep(2) polls of a ready flag before a persistent chain gives up (about a second)
constexpr int kReadySpins = 1 << 24;

template <int D, bool BF16, int CW>
struct ChainSmem {
  using Gm = Geo<D, BF16>;
  static constexpr size_t KQ = Gm::KQ_BYTES;                       // Q tiles of the k-head
  static constexpr size_t HT = Gm::HT_TILES * kTileBytes;          // -W, K^T decayed, P of the v-head
  static constexpr size_t VW = CW * 4 * Pk<BF16>::VC_BYTES;        // U' tiles of this workgroup's rows
  static constexpr size_t GATES = Gm::GATE_BYTES;
  static constexpr size_t BYTES = KQ + HT + VW + GATES;
  // loader waves: 4 where every segment of the buffer is a multiple of 4 KB, else 2
  static constexpr int NKQ = static_cast<int>(KQ / 1024), NHT = static_cast<int>(HT / 1024);
  static constexpr int NVW = static_cast<int>(VW / 1024);
  static constexpr int NL = (NKQ % 4 == 0 && NHT % 4 == 0 && NVW % 4 == 0) ? 4 : 2;
  // 1 KB blocks: the segments above plus one block for the gates
  static constexpr size_t BUF = static_cast<size_t>(NKQ + NHT + NVW + 1) * 1024;
  static_assert(2 * BUF <= 150 * 1024, "two chunk buffers must fit in LDS");
};

// Workgroup -> (sequence, v-head, block of CW x 16 rows of d_v).  Workgroups
// are dispatched to the 8 XCDs round robin by linear id; the logical index
// q = (s * Hv + h) * Z + z is spread so that consecutive q (the workgroups of
// one k-head, which read the same Q tiles, and of one v-head, which read the
// same W, K^T and P tiles) share an XCD and its L2.
__device__ __forceinline__ int chain_logical_index(int L, int nwg) {
  return (nwg % 8 == 0) ? (L % 8) * (nwg / 8) + L / 8 : L;
}

// One sequence as a chain launch sees it: the sequence's chunks in [c0,
// c0 + ncl) of the chunk table are this launch's; the state carries over
// between launches through the slot (fp32, exact).  A sequence without chunks
// belongs to the launch that starts at chunk 0.  False: nothing to do here.
struct ChainSeq {
  bool init, seq_last, state_in;
  int slot, seq_start, len, c0, cr0, ncl, ckpt0;
  uint32_t pos0;
};
__device__ __forceinline__ bool chain_seq(const PrefillArgs& A, const PrefillLayout& Lay, int s, ChainSeq& q) {
  const int32_t* se = ws_ptr<int32_t>(A.workspace, Lay.seq_tab) + 8 * s;
  if (!(se[SQ_FLAGS] & SQF_VALID)) return false;
  const int first = se[SQ_FIRST], nc = se[SQ_NCHUNK];
  const int c0 = max(first, A.seg_lo), c1 = min(first + nc, A.seg_hi);
  if (nc == 0 ? A.seg_lo != 0 : c0 >= c1) return false;
  const bool seq_first = nc == 0 || c0 == first;  // the sequence starts in this launch
  q.init = (se[SQ_FLAGS] & SQF_INIT) != 0;
  q.seq_last = nc == 0 || c1 == first + nc;       // ... and ends in it
  q.state_in = seq_first ? q.init : true;
  q.slot = se[SQ_SLOT];
  q.seq_start = se[SQ_START];
  q.len = se[SQ_LEN];
  q.c0 = c0;
  q.cr0 = c0 - first;
  q.ncl = c1 - c0;
  q.pos0 = static_cast<uint32_t>(se[SQ_POS0]);
  q.ckpt0 = se[SQ_CKPT0];
  return true;
}

// Chain workgroup: CW compute waves (wave w holds rows 16 (z CW + w) ..) and
// kLoaders loader waves.  While the compute waves work on chunk c from one
// LDS buffer, the loaders copy chunk c+1 (the Q tiles of the k-head, the -W /
// K^T / P tiles of the v-head, this workgroup's U' tiles and the gate factors)
// into the other; one workgroup barrier per chunk swaps the buffers.  The
// waves of a workgroup sit on different SIMDs, so the copies cost the
// compute waves no issue slots.
template <int D, bool BF16, int CW>
__global__ __launch_bounds__((CW + ChainSmem<D, BF16, CW>::NL) * 64, 1) void chain_kernel(PrefillArgs A, PrefillLayout Lay) {
  using P = Pk<BF16>;
  using Gm = Geo<D, BF16>;
  using Sm = ChainSmem<D, BF16, CW>;
  using Ch = Chain<BF16>;
  using E = typename P::E;
  using Bop = typename Ch::Bop;
  constexpr int KSD = Gm::KSD, KSC = Gm::KSC, NT = Gm::NT, TPS = Gm::TPS, Z = NT / CW;
  __shared__ __attribute__((aligned(1024))) char lds0[Sm::BUF];
  __shared__ __attribute__((aligned(1024))) char lds1[Sm::BUF];

  const int q = chain_logical_index(blockIdx.x, gridDim.x);
  const int zb = q % Z, h = (q / Z) % A.Hv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int dvt = zb * CW + wave;                // a compute wave's 16 rows of d_v
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk, kh = h / G;
  const int g = lane >> 4, col = lane & 15;
  // A persistent launch has one workgroup per (v-head, row block) that walks
  // the sequences in table order, the order in which the chunk kernel
  // publishes their chunks; a segment launch has one workgroup per sequence
  // as well.  Loader and compute waves walk the same sequences and take the
  // same barriers for each; at the end of a sequence the loaders write the
  // q|k channels of its conv history and the compute waves the v channels.
  const int s_lo = A.persistent ? 0 : q / (Z * A.Hv);
  const int s_hi = A.persistent ? A.n_seqs : s_lo + 1;

  // ---- loader waves: two chunks in flight in registers ----
  if (wave >= CW) {
    for (int s = s_lo; s < s_hi; ++s) {
      ChainSeq sq;
      if (!chain_seq(A, Lay, s, sq)) continue;
      const bool init = sq.init, seq_last = sq.seq_last;
      const int slot = sq.slot, seq_start = sq.seq_start, len = sq.len, c0 = sq.c0, ncl = sq.ncl;
      const uint32_t pos0 = sq.pos0;
      constexpr int NL = Sm::NL;
      const int lw = wave - CW;
      const char* wsb = static_cast<const char*>(A.workspace);
      // 1 KB blocks [Q | -W, K^T, P | U' | gates]; loader lw copies blocks
      // NL j + lw.  Every segment starts at a multiple of NL blocks, so the
      // segment of round j is known at compile time.
      constexpr int NKQ = Sm::NKQ, NHT = Sm::NHT, NVW = Sm::NVW, NBLK = NKQ + NHT + NVW + 1;
      constexpr int NJ = (NBLK + NL - 1) / NL;
      static_assert(NKQ % NL == 0 && NHT % NL == 0 && NVW % NL == 0 && Sm::VW % 1024 == 0, "segment alignment");
      static_assert(Sm::GATES <= 1024, "gates fit one block");
      static_assert(NBLK * 1024 == static_cast<int>(Sm::BUF), "blocks fill the buffer");
      // Both register sets are always filled (a chunk past the end reloads the
      // last chunk into unused registers), so their accesses stay unconditional.
      const int clast = c0 + (ncl > 0 ? ncl - 1 : 0);
      // In a persistent launch the chunk kernel runs concurrently: wait until it
      // has published (chunk, kh).  The flag is read with an agent-scope atomic
      // (it bypasses this XCD's L2); the operand lines read after it were not
      // touched earlier by this kernel, so they come from memory.  The wait is
      // bounded: on time-out the error word is set and the loader goes on.
      const int32_t* ready = ws_ptr<int32_t>(A.workspace, Lay.ready);
      bool timed_out = false;
      auto wait_ready = [&](int chunk) {
        if (!A.persistent || timed_out) return;
        const int32_t* f = ready + chunk * Hk + kh;
        for (int spins = 0; __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > kReadySpins) {
            report_error(A.dev_err, GDN_DEV_WAIT_TIMEOUT);
            timed_out = true;
            break;
          }
        }
      };
      auto fetch = [&](uint4 (&r)[NJ], int chunk) {
        chunk = min(chunk, clast);
        wait_ready(chunk);
        const char* kq = wsb + Lay.kq + (static_cast<size_t>(chunk) * Hk + kh) * Gm::KQ_BYTES;
        const char* hb = wsb + Lay.head + (static_cast<size_t>(chunk) * Hv + h) * Gm::HEAD_BYTES;
        const char* vwb = hb + Gm::VW_OFF + static_cast<size_t>(zb) * CW * 4 * P::VC_BYTES;
        // an opaque copy of this lane's offset keeps the compiler from hoisting
        // one address register per block out of the chunk loop
        int lo = lw * 1024 + lane * 16;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int b0 = j * NL;                     // first block of this round
          const char* src;
          if (b0 < NKQ) src = kq + b0 * 1024;
          else if (b0 < NKQ + NHT) src = hb + (b0 - NKQ) * 1024;
          else if (b0 < NKQ + NHT + NVW) src = vwb + (b0 - NKQ - NHT) * 1024;
          else src = hb + Gm::GATE_OFF - lw * 1024;  // gates: loader 0, lanes < GATES / 16
          r[j] = (b0 + NL <= NKQ + NHT + NVW || (lw == 0 && lane * 16 < static_cast<int>(Sm::GATES)))
                     ? *reinterpret_cast<const uint4*>(src + lo)
                     : make_uint4(0, 0, 0, 0);
        }
      };
      auto put = [&](const uint4 (&r)[NJ], char* base) {
        int lo = lw * 1024 + lane * 16;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          if (j + 1 < NJ || lw == 0) *reinterpret_cast<uint4*>(base + j * NL * 1024 + lo) = r[j];
      };
      // Before barrier i the buffer (i % 2) holds chunk c0 + i; chunk i+1 and
      // i+2 are in flight in the two register sets meanwhile.
      uint4 ra[NJ], rb[NJ];
      if (ncl > 0) {  // a sequence without chunks stages nothing (its chunk index may be past the table)
        fetch(ra, c0);
        fetch(rb, c0 + 1);
        put(ra, lds0);
      }
      lds_barrier();
      if (ncl > 0) fetch(ra, c0 + 2);
      for (int ci = 0; ci < ncl; ci += 2) {
        put(rb, lds1);            // chunk ci + 1 (past the end: never read)
        lds_barrier();
        fetch(rb, c0 + ci + 3);
        if (ci + 1 < ncl) {
          put(ra, lds0);          // chunk ci + 2
          lds_barrier();
          fetch(ra, c0 + ci + 4);
        }
      }
      // ---- conv history: the last W-1 inputs go to ring rows pos_end-1 .. pos_end-W+1 ----
      if (A.W > 0 && seq_last) {
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
        if (h % G == 0 && zb == 0)
          for (int cc = tid - CW * 64; cc < 2 * D; cc += Sm::NL * 64) put(cc < D ? kh * D + cc : Hk * D + kh * D + (cc - D));
      }
    }  // sequences
  } else {
    for (int s = s_lo; s < s_hi; ++s) {
      ChainSeq sq;
      if (!chain_seq(A, Lay, s, sq)) continue;
      const bool init = sq.init, seq_last = sq.seq_last, state_in = sq.state_in;
      const int slot = sq.slot, seq_start = sq.seq_start, len = sq.len, cr0 = sq.cr0, ncl = sq.ncl;
      const int ckpt0 = sq.ckpt0;
      const uint32_t pos0 = sq.pos0;
      float* Sglob = A.state + (static_cast<size_t>(slot) * Hv + h) * D * D + static_cast<size_t>(16 * dvt + col) * D;

      // ---- compute waves: S^T slice in accumulators, tile i holds S^T[16i + 4g + e][16 dvt + col] ----
      f32x4_t st[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (state_in) {
          const float4 v = *reinterpret_cast<const float4*>(Sglob + 16 * i + 4 * g);
          st[i] = f32x4_t{v.x, v.y, v.z, v.w};
        } else {
          st[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }

      // One chunk step from an LDS buffer; O returned in registers.  The body
      // runs in stages separated by scheduling barriers: every stage issues the
      // LDS reads of the operand tiles the NEXT stage multiplies, so those reads
      // are in flight while this stage's MFMAs run (a wave has no other wave on
      // its SIMD to hide LDS latency behind).
      auto compute = [&](const char* base, f32x4_t (&O)[4]) {
        const uint4* qa = reinterpret_cast<const uint4*>(base);
        const uint4* ht = reinterpret_cast<const uint4*>(base + Sm::KQ);
        const E* vw = reinterpret_cast<const E*>(base + Sm::KQ + Sm::HT) + wave * 4 * 256;
        const float* gt = reinterpret_cast<const float*>(base + Sm::KQ + Sm::HT + Sm::VW);
        auto tile = [&](const uint4* arr, int t) { return arr[t * 64 + lane]; };
        auto fence = [] {
#if GDN_CHAIN_SCHED
          __builtin_amdgcn_sched_barrier(0);
#endif
        };

        // stage 0: -W tiles, U', e^{G_last}
        uint4 wa[4][KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) wa[mt][ks] = tile(ht + Gm::WA * 64, mt * KSD + ks);
        f32x4_t U[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if constexpr (BF16) {
            const uint2 r2 = *reinterpret_cast<const uint2*>(vw + mt * 256 + lane * 4);
            U[mt] = f32x4_t{__uint_as_float(r2.x << 16), __uint_as_float(r2.x & 0xffff0000u),
                            __uint_as_float(r2.y << 16), __uint_as_float(r2.y & 0xffff0000u)};
          } else {
            const float4 r4 = *reinterpret_cast<const float4*>(vw + mt * 256 + lane * 4);
            U[mt] = f32x4_t{r4.x, r4.y, r4.z, r4.w};
          }
        }
        const float eGl = gt[kC];
        // B operands of S^T (d_k in packed order)
        Bop bS[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int i0 = ks * TPS;
          bS[ks] = Ch::bop(st[i0], (TPS == 2 && i0 + 1 < NT) ? st[(i0 + 1) % NT] : f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
        fence();
        // stage 1: U = U' - W S^T; read the Q tiles
        uint4 qt[4][KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) qt[mt][ks] = tile(qa, mt * KSD + ks);
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) U[mt] = Ch::step(wa[mt][ks], bS[ks], U[mt]);
        fence();
        // stage 2: Y = Q S^T, S^T scaled by e^{G_last}; read the decayed K^T tiles
        uint4 kd[NT][KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
          for (int i = 0; i < NT; ++i) kd[i][ks] = tile(ht + Gm::KDA * 64, i * KSC + ks);
        f32x4_t Y[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Y[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) Y[mt] = Ch::step(qt[mt][ks], bS[ks], Y[mt]);
#pragma unroll
        for (int i = 0; i < NT; ++i) st[i] = st[i] * eGl;
        Bop bU[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) bU[ks] = Ch::bop(U[ks * TPS], U[(ks * TPS + 1) % 4]);
        fence();
        // stage 3: S^T <- e^{G_last} S^T + (diag(e^{G_last - G}) K)^T U; read the P tiles and e^G
        uint4 pt[4][KSC];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
            if (ks * P::SK < 16 * (mt + 1)) pt[mt][ks] = tile(ht + Gm::PA * 64, mt * KSC + ks);
        float4 eg[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) eg[mt] = *reinterpret_cast<const float4*>(gt + 16 * mt + 4 * g);
#pragma unroll
        for (int ip = 0; ip < NT; ip += 2)
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
            for (int i = ip; i < ip + 2 && i < NT; ++i) st[i] = Ch::step(kd[i][ks], bU[ks], st[i]);
        fence();
        // stage 4: O = diag(e^G) Y + P U
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4_t o = Y[mt] * f32x4_t{eg[mt].x, eg[mt].y, eg[mt].z, eg[mt].w};
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
            if (ks * P::SK < 16 * (mt + 1)) o = Ch::step(pt[mt][ks], bU[ks], o);
          O[mt] = o;
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

      // State checkpoint after chunk ci of the sequence when its end is a
      // multiple of ckpt_every tokens (a partial last chunk never is one); the
      // same layout and store pattern as the final state.
      auto store_ckpt = [&](int ci) {
        if (A.ckpt_every <= 0) return;
        const int done = kC * (ci + 1);
        if (done > len || done % A.ckpt_every != 0) return;
        float* cb = A.ckpt + (static_cast<size_t>(ckpt0 + done / A.ckpt_every - 1) * Hv + h) * D * D +
                    static_cast<size_t>(16 * dvt + col) * D;
#pragma unroll
        for (int i = 0; i < NT; ++i)
          *reinterpret_cast<float4*>(cb + 16 * i + 4 * g) = make_float4(st[i][0], st[i][1], st[i][2], st[i][3]);
      };

      {
        f32x4_t O[4];
        lds_barrier();  // the first chunk staged
        for (int ci = 0; ci < ncl; ci += 2) {
          if (ci > 0) store_o(cr0 + ci - 1, O);
          compute(lds0, O);
          store_ckpt(cr0 + ci);
          lds_barrier();
          if (ci + 1 < ncl) {
            store_o(cr0 + ci, O);
            compute(lds1, O);
            store_ckpt(cr0 + ci + 1);
            lds_barrier();
          }
        }
        if (ncl > 0) store_o(cr0 + ncl - 1, O);
      }

      // ---- final state back to the slot ----
#pragma unroll
      for (int i = 0; i < NT; ++i)
        *reinterpret_cast<float4*>(Sglob + 16 * i + 4 * g) = make_float4(st[i][0], st[i][1], st[i][2], st[i][3]);
      // ---- conv history: the last W-1 inputs go to ring rows pos_end-1 .. pos_end-W+1 ----
      if (A.W > 0 && seq_last) {
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
        if (lane < 16) put(2 * Hk * D + h * D + 16 * dvt + lane);
        if (h == 0 && zb == 0 && tid == 0) A.conv_pos[slot * kPosStride] = static_cast<int32_t>(pos_end << kPosShift);
      }
    }  // sequences
  }
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------
// Chunks per launch segment: the workspace of one segment (about 4.4 MB per
// chunk at 16 k-heads / 48 v-heads / d = 128) stays resident in the 256 MB
// last-level cache between the chunk kernel that writes it and the chain
// kernel that reads it.
constexpr int kSegChunks = 16;

// The chain of segment k runs on a second stream of the library while the
// chunk kernel of segment k+1 runs on the caller's stream: the two use
// different compute units (the chain is latency-bound on a fraction of the
// chip, the chunk kernel fills the rest).  One auxiliary stream and a few
// events per device are created on the first prefill call on that device and
// kept for the life of the process; the call joins the auxiliary stream back
// into the caller's stream before it returns, so the caller sees every
// kernel of the call ordered on its own stream.  The single-launch form
// needs the chain and chunk kernels resident at the same time (the chain
// waits on flags the chunk kernel sets, with a bounded wait), so the prefill
// is meant for direct launches, not for replay from a captured graph.
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t ev[8] = {};
};
static std::mutex g_aux_mu;
static AuxStream g_aux[64];

static int aux_stream(AuxStream** out) {
  int dev = 0;
  int e = static_cast<int>(hipGetDevice(&dev));
  if (e) return e;
  if (dev < 0 || dev >= 64) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_aux_mu);
  AuxStream& x = g_aux[dev];
  if (!x.s) {
    hipStream_t st = nullptr;
    e = static_cast<int>(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
    if (e) return e;
    for (hipEvent_t& ev : x.ev) {
      e = static_cast<int>(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
      if (e) return e;
    }
    x.s = st;
  }
  *out = &x;
  return 0;
}

// Largest chain grid that runs as one launch beside the chunk kernel (half the
// CUs: the rest stay free for chunk workgroups, which never wait).
constexpr int kPersistentChainMax = 128;

template <int D, bool BF16>
static int launch_prefill_fit(const PrefillArgs& a0, hipStream_t st) {
  constexpr int CWMAX = BF16 ? 4 : 2;
  constexpr int CW = Geo<D, BF16>::NT < CWMAX ? Geo<D, BF16>::NT : CWMAX;
  const PrefillLayout L = layout_t<D, BF16>(a0.Hk, a0.Hv, a0.max_chunks, a0.n_seqs);
  AuxStream* aux = nullptr;
  int e = aux_stream(&aux);
  if (e) return e;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, a0, L);
  e = static_cast<int>(hipGetLastError());
  if (e) return e;
  const size_t smem = ChunkSmem<D, BF16>::BYTES;
  auto chunk_fn = a0.W == 4 ? &chunk_kernel<D, BF16, 4> : &chunk_kernel<D, BF16, 0>;
  e = static_cast<int>(hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fn),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem)));
  if (e) return e;
  const int chain_wgs_seq = a0.Hv * (Geo<D, BF16>::NT / CW);  // chain workgroups per sequence
  const dim3 chain_block((CW + ChainSmem<D, BF16, CW>::NL) * 64);
  if (chain_wgs_seq <= kPersistentChainMax && a0.max_chunks <= 65535) {  // 65535: grid y limit
    // One chain launch over all sequences in turn, beside one chunk launch
    // over all chunks: the chain's loaders wait on each (chunk, k-head) flag.
    // The chain grid holds at most half the CUs, so chunk workgroups always
    // find CUs.
    const int chain_wgs = chain_wgs_seq;
    PrefillArgs a = a0;
    a.persistent = 1;
    a.seg_lo = 0;
    a.seg_hi = a0.max_chunks;
    e = static_cast<int>(hipEventRecord(aux->ev[0], st));  // after the plan
    if (e) return e;
    e = static_cast<int>(hipStreamWaitEvent(aux->s, aux->ev[0], 0));
    if (e) return e;
    hipLaunchKernelGGL((chain_kernel<D, BF16, CW>), dim3(chain_wgs), chain_block, 0, aux->s, a, L);
    e = static_cast<int>(hipGetLastError());
    if (e) return e;
    if (a0.max_chunks > 0) {
      hipLaunchKernelGGL(chunk_fn, dim3(a.Hk, a0.max_chunks), dim3(kChunkThreads), smem, st, a, L);
      e = static_cast<int>(hipGetLastError());
      if (e) return e;
    }
  } else {
    const int chain_wgs = a0.n_seqs * chain_wgs_seq;
    // at least one segment, so that sequences without tokens still get their slot written
    int seg = 0;
    for (int lo = 0; lo == 0 || lo < a0.max_chunks; lo += kSegChunks, ++seg) {
      PrefillArgs a = a0;
      a.seg_lo = lo;
      a.seg_hi = lo + kSegChunks;
      const int n = a0.max_chunks - lo < kSegChunks ? a0.max_chunks - lo : kSegChunks;
      if (n > 0) {
        hipLaunchKernelGGL(chunk_fn, dim3(a.Hk, n), dim3(kChunkThreads), smem, st, a, L);
        e = static_cast<int>(hipGetLastError());
        if (e) return e;
      }
      // the chain of this segment waits for its chunk kernel (and, through the
      // caller's stream order, for the plan and every earlier chunk kernel)
      hipEvent_t ready = aux->ev[1 + seg % 6];
      e = static_cast<int>(hipEventRecord(ready, st));
      if (e) return e;
      e = static_cast<int>(hipStreamWaitEvent(aux->s, ready, 0));
      if (e) return e;
      hipLaunchKernelGGL((chain_kernel<D, BF16, CW>), dim3(chain_wgs), chain_block, 0, aux->s, a, L);
      e = static_cast<int>(hipGetLastError());
      if (e) return e;
    }
  }
  e = static_cast<int>(hipEventRecord(aux->ev[7], aux->s));
  if (e) return e;
  return static_cast<int>(hipStreamWaitEvent(st, aux->ev[7], 0));
}

template <int D, bool BF16>
static int launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  if constexpr (ChunkSmem<D, BF16>::BYTES > 160 * 1024) {
    return static_cast<int>(hipErrorInvalidValue);  // refused by the API before any launch
  } else {
    return launch_prefill_fit<D, BF16>(a, st);
  }
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
