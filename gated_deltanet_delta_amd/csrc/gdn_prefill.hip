// Chunked (WY / UT-transform) prefill of the gated delta rule on gfx950.
//
// Inside a chunk of n <= 64 tokens of one sequence, with cumulative log-gates
// G_r = sum_{j<=r} g_j and the state S at the chunk start (d_v x d_k):
//   L_rj = beta_r e^{G_r - G_j} (k_r . k_j)   for r > j (0 otherwise)
//   T    = (I + L)^{-1}                              (unit lower triangular)
//   U    = T diag(beta) (V - diag(e^G) K S^T)        (the corrected writes u_r)
//   O    = diag(e^G) Q S^T + P U,  P_rj = e^{G_r - G_j} (q_r . k_j) for j <= r
//   S   <- e^{G_last} S + U^T diag(e^{G_last - G}) K
// This is an exact reorganisation of the token-by-token rule (it follows from
// unrolling S_r = alpha_r S_{r-1} + u_r k_r^T inside the chunk).  Every
// exponent is a difference G_r - G_j with r >= j (or G_r itself), so it is
// <= 0 and nothing overflows.  The state after token r inside the chunk is
// e^{G_r} S + U^T diag(d^(r)) K with d^(r)_j = e^{G_r - G_j} for j <= r and 0
// after, which gives state checkpoints at any token.
//
// Two kernels per call, both on the caller's stream:
//   plan:    one workgroup turns the device cu_seqlens into a sequence table
//            and clears the hand-off flags and counters -- no host sync;
//   prefill: one launch of one workgroup per CU (8 per XCD round robin:
//            workgroup b runs on XCD b % 8).  Every workgroup reads the id of
//            the XCD it runs on and takes a ticket from that XCD's counter.
//            All the work of a k-head stays on one XCD, so everything passed
//            between workgroups goes through that XCD's L2:
//            - the first tickets are chain workgroups, one per (v-head, column
//              group) of the XCD's k-heads.  A chain workgroup first produces
//              one of the earliest items (below), then walks every sequence's
//              chunks in order and keeps its columns of the v-head's state S^T
//              in MFMA accumulators from the first chunk of a sequence to its
//              last; per chunk it does what depends on the state: K S^T, U,
//              Q S^T, P U and the state update.  Its helper waves stage the
//              next chunk's operands into LDS and store the output.
//            - the other workgroups are producers: they take (chunk, k-head)
//              items in chunk order and compute what does not depend on the
//              state -- conv + SiLU of q, k and v, the L2 norms of q and k, the
//              gates and their cumulative sums, K K^T and K Q^T on MFMA, then
//              per v-head P and T diag(beta) with T = (I + L)^{-1} -- written
//              pre-packed in MFMA operand order into a ring of chunk slots.
//            A producer publishes (chunk, k-head) with a flag once its stores
//            have reached the L2; a chain workgroup marks a chunk consumed once
//            it sits in LDS, and a producer reuses a ring slot only after every
//            chain workgroup of its k-head has consumed the chunk it held.
//
// Forward progress.  A workgroup takes its ticket only while it runs, and the
// first tickets of every XCD are the chain roles, so every chain workgroup is
// resident before any producer exists.  Chain workgroups wait only on items
// published by producers (the one item a chain workgroup produces first lies
// in a chunk below the ring depth, so it waits for nothing); a producer
// waits only on the chain having consumed
// a chunk RING slots older than its own.  Items are taken in chunk order by
// running workgroups, so the producer of the oldest unpublished item is always
// resident and its wait is always on already published chunks: the chain can
// reach it, and the launch drains.  Every wait is bounded (about a second);
// on time-out the error word gets GDN_DEV_WAIT_TIMEOUT, an abort word ends
// every other wait, and the launch still finishes.  The last workgroup out
// checks that every chain role and every item was done (GDN_DEV_INCOMPLETE
// otherwise), so no dispatch pattern can leave outputs silently unwritten.
//
// Packed operand tiles.  A 16 x SK sub-matrix (rows r, contraction index k;
// SK = 32 for the bf16 MFMA 16x16x32, 16 for four fp32 MFMA 16x16x4) is
// stored as 64 lanes x 16 bytes.  Lane (g = k%16 / 4) * 16 + r holds, in
// element e = (k / 16) * 4 + k % 4, the value at (r, k).  A 16x16
// accumulator tile holds rows 4g..4g+3 of column l%16 in lane l, so the
// accumulators of tiles (2s, 2s+1) (bf16) or tile s (fp32) form exactly the
// B operand that pairs with packed tile column s -- and, read the other way,
// the packed A tile of the transposed product.
#include <type_traits>

#include <mutex>

#include <hip/hip_ext.h>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kC = kChunk;             // 64 tokens per chunk
constexpr int kMaxGroup = 8;           // v-heads per k-head
constexpr int kLd = kC + 1;            // row stride of 64x64 fp32 matrices in LDS
constexpr int kTileBytes = 1024;
constexpr int kThreads = 512;          // 8 waves in every workgroup, whatever its role
constexpr int kWaves = kThreads / 64;
constexpr int kXcd = 8;                // XCDs of the chip; workgroup b is dispatched to XCD b % 8
constexpr int kWgPerXcd = 32;          // one workgroup per CU
constexpr int kMaxChainPerXcd = 24;    // chain workgroups per XCD and launch; the rest produce
constexpr int kRingSlots = 16;         // chunks a producer may run ahead of the chain
constexpr int kLine = 32;              // int32 words per 128-byte line
constexpr int kSpins = 1 << 24;        // s_sleep(2) polls before a wait gives up (about a second)
constexpr size_t kLdsStageMax = 156 * 1024;  // two chain stages above this: one buffer
constexpr int kCtrLines = 2 * kXcd + 1;     // per launch: role and item ticket per XCD, exit word

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

template <bool BF16>
struct Pk {
  using E = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int SK = BF16 ? 32 : 16;         // contraction length of one packed tile
  static constexpr int EPL = BF16 ? 8 : 4;          // elements per lane (16 bytes)
  static constexpr int VC_BYTES = 256 * sizeof(E);  // one 16x16 tile in accumulator layout
};

// The packed tiles of a lower-triangular 64x64 matrix that are not
// identically zero: (row tile ti, packed column ks) with ks * SK <= 16 ti + 15,
// numbered row tile by row tile.
template <bool BF16>
struct TriTiles {
  static constexpr int SK = Pk<BF16>::SK;
  static constexpr int per_row(int ti) { return (16 * ti + 15) / SK + 1; }
  static constexpr int count() { return per_row(0) + per_row(1) + per_row(2) + per_row(3); }
  static constexpr int index(int ti, int ks) {
    int n = 0;
    for (int t = 0; t < ti; ++t) n += per_row(t);
    return n + ks;
  }
  __device__ static void at(int t, int& ti, int& ks) {
    ti = 0;
    while (t >= per_row(ti)) { t -= per_row(ti); ++ti; }
    ks = t;
  }
};

// A v-head's chain runs as NCG workgroups, each owning NT / NCG 16-row tiles
// of d_v (the columns of S^T): every product of the chain splits along d_v
// with no exchange between them.  At d = 128 (bf16) there are two, so that a
// compute wave holds one tile: its chunk step is shorter, and the chain with
// checkpoints fits the registers.
template <int D, bool BF16>
constexpr int ncg_of() { return (D == 128 && BF16) ? 2 : 1; }

template <int D, bool BF16, int NCG_ = 1>
struct Geo {
  using P = Pk<BF16>;
  static constexpr int KSD = (D + P::SK - 1) / P::SK;  // packed tiles along d
  static constexpr int KSC = kC / P::SK;               // packed tiles along the chunk
  static constexpr int NT = D / 16;                    // 16-row tiles along d
  static constexpr int TPS = P::SK / 16;               // accumulator tiles per packed super-step
  static constexpr int NTRI = TriTiles<BF16>::count();
  // One ring item (chunk, k-head), in 1 KB tiles:
  static constexpr int QA = 0;                 // Q as A (rows token, k = d): 4 x KSD
  static constexpr int KA = 4 * KSD;           // K as A (rows token, k = d): 4 x KSD
  static constexpr int KT = 8 * KSD;           // K^T as A (rows d, k = token): NT x KSC
  static constexpr int HEAD0 = 8 * KSD + NT * KSC;
  // then per v-head of the group: T diag(beta) and P as A (NTRI tiles each),
  // gates (1 tile), and V in accumulator layout (tile (d_v / 16, token / 16),
  // lane (token % 16 / 4) * 16 + d_v % 16, element token % 4; NV tiles of 1 KB)
  static constexpr int NV = NT * 4 * P::VC_BYTES / kTileBytes;
  static constexpr int HT = 0, HP = NTRI, HG = 2 * NTRI, HV = 2 * NTRI + 1, HEAD_TILES = HV + NV;
  // gate tile: e^G [64], e^{G_last - G} [64], G [64], e^{G_last} (64 copies)
  static constexpr int G_EG = 0, G_D = 64, G_G = 128, G_EGL = 192;
  static constexpr int NCG = NCG_;
  static constexpr int NTG = NT / NCG;                 // d_v tiles of one chain workgroup
  static constexpr int NVG = NV / NCG;                 // its V tiles (contiguous: tile-major in d_v)
  // A chain stage in LDS: the item's shared tiles, then one head's T, P and
  // gate tiles, then the workgroup's V tiles
  static constexpr int STAGE_TILES = HEAD0 + HV + NVG;
  static constexpr size_t V_OFF = static_cast<size_t>(HEAD0 + HV) * kTileBytes;
  static constexpr size_t STAGE_BYTES = static_cast<size_t>(STAGE_TILES) * kTileBytes;
  static constexpr int NBUF = 2 * STAGE_BYTES <= kLdsStageMax ? 2 : 1;
  // chain compute waves: CT 16-row tiles of d_v each
  static constexpr int CT = NCG > 1 ? 1 : (NT >= 2 ? 2 : 1);
  static constexpr int NWC = NTG / CT;
  static size_t item_bytes(int G) { return static_cast<size_t>(HEAD0 + G * HEAD_TILES) * kTileBytes; }
};

// Sequence s needs ceil(len_s / C) chunks, and the sum of those is at most
// floor((n_tokens + (C - 1) n_seqs) / C).
int prefill_max_chunks(int n_tokens, int n_seqs) {
  return static_cast<int>((static_cast<int64_t>(n_tokens) + static_cast<int64_t>(kC - 1) * n_seqs) / kC);
}

// k-heads of one launch: 8 XCDs x as many k-heads per XCD as keep the chain
// workgroups of an XCD (G x NCG per k-head) within kMaxChainPerXcd.
static int heads_per_launch(int Hk, int Hv, int ncg) {
  const int per_head = (Hv / Hk) * ncg;
  const int per_xcd = kMaxChainPerXcd / per_head > 0 ? kMaxChainPerXcd / per_head : 1;
  return kXcd * per_xcd;
}

static int launches(int Hk, int Hv, int ncg) {
  const int n = heads_per_launch(Hk, Hv, ncg);
  return (Hk + n - 1) / n;
}

int prefill_launches(int Hk, int Hv, int D, bool bf16) {
  return launches(Hk, Hv, (D == 128 && bf16) ? ncg_of<128, true>() : 1);
}

template <int D, bool BF16>
static PrefillLayout layout_t(int Hk, int Hv, int n_tokens, int S) {
  using Gm = Geo<D, BF16>;
  PrefillLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
  const int maxc = prefill_max_chunks(n_tokens, S);
  L.ring_slots = maxc < 1 ? 1 : (maxc < kRingSlots ? maxc : kRingSlots);
  L.item_bytes = Gm::item_bytes(Hv / Hk);
  L.ring = take(static_cast<size_t>(L.ring_slots) * Hk * L.item_bytes);
  L.hdr = take(2 * kLine * 4);
  L.seq_tab = take(static_cast<size_t>(S) * 8 * 4);
  L.ready = take(static_cast<size_t>(L.ring_slots) * Hk * kLine * 4);
  L.consumed = take(static_cast<size_t>(Hv) * ncg_of<D, BF16>() * kLine * 4);
  L.ctr = take(static_cast<size_t>(launches(Hk, Hv, ncg_of<D, BF16>())) * kCtrLines * kLine * 4);
  L.total = off;
  return L;
}

PrefillLayout prefill_layout(int Hk, int Hv, int D, bool bf16, int n_tokens, int S) {
  switch (D) {
    case 16: return bf16 ? layout_t<16, true>(Hk, Hv, n_tokens, S) : layout_t<16, false>(Hk, Hv, n_tokens, S);
    case 32: return bf16 ? layout_t<32, true>(Hk, Hv, n_tokens, S) : layout_t<32, false>(Hk, Hv, n_tokens, S);
    case 64: return bf16 ? layout_t<64, true>(Hk, Hv, n_tokens, S) : layout_t<64, false>(Hk, Hv, n_tokens, S);
    default: return bf16 ? layout_t<128, true>(Hk, Hv, n_tokens, S) : layout_t<128, false>(Hk, Hv, n_tokens, S);
  }
}

// Sequence table entry (int32 x 8).  SQ_CKPT0: index of the sequence's first
// state checkpoint.
enum { SQ_FIRST = 0, SQ_NCHUNK, SQ_POS0, SQ_FLAGS, SQ_SLOT, SQ_START, SQ_LEN, SQ_CKPT0 };
enum { SQF_VALID = 1, SQF_INIT = 2 };
enum { HDR_TOTAL = 0, HDR_ABORT = kLine };

template <typename T>
__device__ __forceinline__ T* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// XCD (XCC) the calling wave runs on, from the hardware register XCC_ID.
__device__ __forceinline__ int xcc_id() {
  return static_cast<int>(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)) & (kXcd - 1));
}

// Bounded wait until *flag >= want.  False on time-out (reported, and the
// abort word set so that every other wait of the call ends) or once another
// wait of the call has timed out.
__device__ __forceinline__ bool wait_at_least(const int32_t* flag, int32_t want, int32_t* abort_word,
                                              int32_t* dev_err) {
  for (int spins = 0;;) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) return true;
    if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return false;
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpins) {
      report_error(dev_err, GDN_DEV_WAIT_TIMEOUT);
      __hip_atomic_store(abort_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
}

// 16-byte load that misses the CU's L1 (cache policy sc0) and is served by
// the XCD's L2: operands another CU of the same XCD published.
__device__ __forceinline__ uint4 load_l2(const void* base, uint32_t off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), static_cast<short>(0), 0x7fffffff, 0x00020000);
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 1);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The same load written straight into LDS (one 1 KB tile per wave: lane i's
// 16 bytes land at lds + 16 i), counted by the wave's vector-memory counter.
__device__ __forceinline__ void load_l2_to_lds(const void* base, uint32_t off, void* lds) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), static_cast<short>(0), 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16, off, 0, 0, 1);
}
// wait for every vector-memory operation of this wave (s_waitcnt vmcnt(0))
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// wait for every LDS operation of this wave (s_waitcnt lgkmcnt(0))
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// ---------------------------------------------------------------------------
// plan: sequence table from cu_seqlens; hand-off state cleared
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(PrefillArgs A, PrefillLayout L, int n_launch) {
  int32_t* stab = ws_ptr<int32_t>(A.workspace, L.seq_tab);
  int32_t* hdr = ws_ptr<int32_t>(A.workspace, L.hdr);
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
    if (total > A.max_chunks) {  // cannot happen for a valid partition
      report_error(A.dev_err, GDN_DEV_BAD_SEQLENS);
      for (int s = 0; s < S; ++s) stab[8 * s + SQ_FLAGS] = 0;
      total = 0;
    }
    hdr[HDR_TOTAL] = total;
    hdr[HDR_ABORT] = 0;
  }
  int32_t* ready = ws_ptr<int32_t>(A.workspace, L.ready);
  for (int i = threadIdx.x; i < L.ring_slots * A.Hk; i += blockDim.x) ready[i * kLine] = 0;
  int32_t* consumed = ws_ptr<int32_t>(A.workspace, L.consumed);
  const int n_cons = static_cast<int>((L.ctr - L.consumed) / (kLine * 4));  // every chain's line
  for (int i = threadIdx.x; i < n_cons; i += blockDim.x) consumed[i * kLine] = 0;
  int32_t* ctr = ws_ptr<int32_t>(A.workspace, L.ctr);
  for (int i = threadIdx.x; i < n_launch * kCtrLines * kLine; i += blockDim.x) ctr[i] = 0;
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
  // b's elements scaled: the first four by d0, the last four by d1
  __device__ static Bop scaled(const Bop& b, const f32x4_t& d0, const f32x4_t& d1) {
    Bop r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r[k] = static_cast<__bf16>(static_cast<float>(b[k]) * d0[k]);
      r[k + 4] = static_cast<__bf16>(static_cast<float>(b[k + 4]) * d1[k]);
    }
    return r;
  }
  // The transposed product: a lane supplies A[row l%16][k-set] and B[k-set][col
  // l%16] in the same register positions, so B-operand registers of X (k, n)
  // are the A operand of X^T (rows n, k) and a packed A tile of Y (rows m, k)
  // is the B operand of Y^T (k, cols m).
  __device__ static f32x4_t step_t(const Bop& a, uint4 b, f32x4_t c) {
    return mfma32(a, __builtin_bit_cast(bf16x8_t, b), c);
  }
};

template <>
struct Chain<false> {
  using Bop = f32x4_t;
  __device__ static Bop bop(const f32x4_t& t0, const f32x4_t&) { return t0; }
  __device__ static Bop scaled(const Bop& b, const f32x4_t& d0, const f32x4_t&) { return b * d0; }
  __device__ static f32x4_t step(uint4 a, const Bop& b, f32x4_t c) {
    c = mfma4(__uint_as_float(a.x), b[0], c);
    c = mfma4(__uint_as_float(a.y), b[1], c);
    c = mfma4(__uint_as_float(a.z), b[2], c);
    return mfma4(__uint_as_float(a.w), b[3], c);
  }
  __device__ static f32x4_t step_t(const Bop& a, uint4 b, f32x4_t c) {
    c = mfma4(a[0], __uint_as_float(b.x), c);
    c = mfma4(a[1], __uint_as_float(b.y), c);
    c = mfma4(a[2], __uint_as_float(b.z), c);
    return mfma4(a[3], __uint_as_float(b.w), c);
  }
};

// 16x16 fp32 tiles as MFMA operands (v_mfma_f32_16x16x4_f32, four steps):
// A row-major at a (stride lda), lane = row (lane & 15); step s contracts
// index 4 s + (lane >> 4).  An accumulator tile (lane: rows 4 (lane >> 4) + i
// of column lane & 15) can be the B operand as it is when its A partner is
// read with step s contracting index 4 (lane >> 4) + s instead ("acc order").
__device__ __forceinline__ f32x4_t tile_a(const float* a, int lda, int lane) {
  f32x4_t v;
#pragma unroll
  for (int s = 0; s < 4; ++s) v[s] = a[(lane & 15) * lda + 4 * s + (lane >> 4)];
  return v;
}
__device__ __forceinline__ f32x4_t tile_a_acc(const float* a, int lda, int lane) {
  f32x4_t v;
#pragma unroll
  for (int s = 0; s < 4; ++s) v[s] = a[(lane & 15) * lda + 4 * (lane >> 4) + s];
  return v;
}
__device__ __forceinline__ f32x4_t tile_b(const float* b, int ldb, int lane) {
  f32x4_t v;
#pragma unroll
  for (int s = 0; s < 4; ++s) v[s] = b[(4 * s + (lane >> 4)) * ldb + (lane & 15)];
  return v;
}
__device__ __forceinline__ f32x4_t mm16(const f32x4_t& a, const f32x4_t& b, f32x4_t acc) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma4(a[s], b[s], acc);
  return acc;
}
__device__ __forceinline__ void settle4(f32x4_t& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ void store16(float* d, int ld, f32x4_t v, float sign, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) d[(4 * (lane >> 4) + i) * ld + (lane & 15)] = sign * v[i];
}

// In-place inverse of the unit lower-triangular I + L (64x64, L strictly lower,
// row stride kLd) by one wave: 16x16 diagonal blocks by forward substitution
// (lane = block x column), then the off-diagonal blocks level by level with
// fp32 MFMA:  [A 0; C B]^-1 = [A^-1 0; -B^-1 C A^-1  B^-1].  Every stage reads
// all its LDS operands before its arithmetic, and each level's inner product
// C A^-1 feeds the outer one from registers.
__device__ __forceinline__ void invert_unit_lower64(float* Lt, int lane) {
  {
    // column by column: once t_j is final, every later row takes its term;
    // the strictly lower triangle of the block is read first
    const int bi = lane >> 4, c = lane & 15;
    float* Lb = Lt + 16 * bi * kLd + 16 * bi;
    float l[16][16];
#pragma unroll
    for (int r = 1; r < 16; ++r)
#pragma unroll
      for (int j = 0; j < r; ++j) l[r][j] = Lb[r * kLd + j];
#pragma unroll
    for (int r = 1; r < 16; ++r)
#pragma unroll
      for (int j = 0; j < r; ++j) settle(l[r][j]);
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = (r == c) ? 1.0f : 0.0f;
#pragma unroll
    for (int j = 0; j < 15; ++j)
#pragma unroll
      for (int r = j + 1; r < 16; ++r) t[r] = fmaf(-l[r][j], t[j], t[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) Lb[r * kLd + c] = t[r];
  }
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  // 32x32 level, diagonal 32-blocks b = 0, 1: T10 = -T11 (L10 T00)
  {
    f32x4_t a[2], bt[2], m[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float* o = Lt + 32 * b * kLd + 32 * b;
      a[b] = tile_a(o + 16 * kLd, kLd, lane);
      bt[b] = tile_b(o, kLd, lane);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      settle4(a[b]);
      settle4(bt[b]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) m[b] = mm16(a[b], bt[b], zero);
#pragma unroll
    for (int b = 0; b < 2; ++b) a[b] = tile_a_acc(Lt + (32 * b + 16) * kLd + 32 * b + 16, kLd, lane);
#pragma unroll
    for (int b = 0; b < 2; ++b) settle4(a[b]);
#pragma unroll
    for (int b = 0; b < 2; ++b) store16(Lt + (32 * b + 16) * kLd + 32 * b, kLd, mm16(a[b], m[b], zero), -1.0f, lane);
  }
  // 64x64 level: T_BA = -T_B (C T_A), 32x32 blocks of 16x16 tiles; C is the
  // lower-left block of L; T_A[0][1] = 0 and T_B[0][1] = 0
  const float* C = Lt + 32 * kLd;
  const float* TB = Lt + 32 * kLd + 32;
  f32x4_t m2[2][2];
  {
    f32x4_t ca[2][2], ta[3];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) ca[rt][kt] = tile_a(C + 16 * rt * kLd + 16 * kt, kLd, lane);
    ta[0] = tile_b(Lt, kLd, lane);                  // T_A[0][0]
    ta[1] = tile_b(Lt + 16 * kLd, kLd, lane);       // T_A[1][0]
    ta[2] = tile_b(Lt + 16 * kLd + 16, kLd, lane);  // T_A[1][1]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) settle4(ca[rt][kt]);
#pragma unroll
    for (int i = 0; i < 3; ++i) settle4(ta[i]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      m2[rt][0] = mm16(ca[rt][1], ta[1], mm16(ca[rt][0], ta[0], zero));
      m2[rt][1] = mm16(ca[rt][1], ta[2], zero);
    }
  }
  {
    f32x4_t tb[3];
    tb[0] = tile_a_acc(TB, kLd, lane);                  // T_B[0][0]
    tb[1] = tile_a_acc(TB + 16 * kLd, kLd, lane);       // T_B[1][0]
    tb[2] = tile_a_acc(TB + 16 * kLd + 16, kLd, lane);  // T_B[1][1]
#pragma unroll
    for (int i = 0; i < 3; ++i) settle4(tb[i]);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      store16(Lt + 32 * kLd + 16 * ct, kLd, mm16(tb[0], m2[0][ct], zero), -1.0f, lane);
      store16(Lt + 48 * kLd + 16 * ct, kLd, mm16(tb[2], m2[1][ct], mm16(tb[1], m2[0][ct], zero)), -1.0f, lane);
    }
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
    for (int i = 0; i < 4; ++i) w[i] = pack2_bf16(f(2 * i), f(2 * i + 1));
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__float_as_uint(f(0)), __float_as_uint(f(1)), __float_as_uint(f(2)), __float_as_uint(f(3)));
  }
}

// ---------------------------------------------------------------------------
// conv + SiLU of two channels over a quarter (16 tokens) of a chunk
// ---------------------------------------------------------------------------
// Where a chunk and its sequence start: the inputs of token t0 + tq - 3 ..
// t0 + tq + 15 (19 rows) are loaded together, clamped into the sequence and
// the chunk so every load is valid; rows before the sequence come from the
// slot's ring (has_init) or are zero.  Tokens at or past the chunk's length
// give zero outputs.  KW = 0: no conv, the input passes through.
struct ChunkPos {
  int t0, len, seq_start, slot;
  uint32_t pos0;
  bool init;
};

template <bool BF16>
struct Rows {
  using RawT = typename std::conditional<BF16, uint32_t, uint2>::type;
  RawT r[19];
  float4 w[2];  // conv weights of the two channels
};

template <bool BF16, int KW>
__device__ __forceinline__ void load_rows(const PrefillArgs& A, int c0, int tq, const ChunkPos& cp, Rows<BF16>& raw) {
  using E = typename Pk<BF16>::E;
  using RawT = typename Rows<BF16>::RawT;
  const E* x = static_cast<const E*>(A.x);
  const int C = A.C;
  if constexpr (KW == 4) {
#pragma unroll
    for (int v = 0; v < 2; ++v) raw.w[v] = *reinterpret_cast<const float4*>(A.conv_w + (c0 + v) * 4);
  }
  const int tfirst = cp.t0 + tq - 3;
  if (tfirst >= cp.seq_start && tq + 16 <= cp.len) {
    const E* xr = x + static_cast<size_t>(tfirst) * C + c0;
#pragma unroll
    for (int i = 0; i < 19; ++i) raw.r[i] = *reinterpret_cast<const RawT*>(xr + static_cast<size_t>(i) * C);
  } else {
#pragma unroll
    for (int i = 0; i < 19; ++i) {
      const int t = min(max(tfirst + i, cp.seq_start), cp.t0 + cp.len - 1);
      raw.r[i] = *reinterpret_cast<const RawT*>(x + static_cast<size_t>(t) * C + c0);
    }
  }
}

template <bool BF16, int KW>
__device__ __forceinline__ void conv_rows(const PrefillArgs& A, int c0, int tq, const ChunkPos& cp,
                                          const Rows<BF16>& raw, float (&y)[2][16]) {
  using RawT = typename Rows<BF16>::RawT;
  const int C = A.C;
  const int tfirst = cp.t0 + tq - 3;
  auto elem = [&](const RawT& r, int v) -> float {
    if constexpr (BF16) return __uint_as_float(v == 0 ? (r << 16) : (r & 0xffff0000u));
    else return __uint_as_float(v == 0 ? r.x : r.y);
  };
  // conv weights times -log2(e): the conv then yields -log2(e) y, the
  // argument the SiLU's exp2 takes
  float w[2][4] = {};
  if constexpr (KW == 4) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const float4 w4 = raw.w[v];
      w[v][0] = kNegLog2e * w4.x; w[v][1] = kNegLog2e * w4.y;
      w[v][2] = kNegLog2e * w4.z; w[v][3] = kNegLog2e * w4.w;
    }
  }
  float hist[2][3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int t = tfirst + i;
#pragma unroll
    for (int v = 0; v < 2; ++v) hist[v][i] = elem(raw.r[i], v);
    if (KW == 4 && t < cp.seq_start) {
      if (cp.init) {
        const float* rr = A.conv_state + (static_cast<size_t>(cp.slot) * A.R +
                                          ring_row(cp.pos0 + static_cast<uint32_t>(t - cp.seq_start), A.R)) * C + c0;
#pragma unroll
        for (int v = 0; v < 2; ++v) hist[v][i] = rr[v];
      } else {
#pragma unroll
        for (int v = 0; v < 2; ++v) hist[v][i] = 0.f;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const float xin = elem(raw.r[3 + r], v);
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
      y[v][r] = tq + r < cp.len ? yy : 0.f;
    }
  }
}

__device__ __forceinline__ ChunkPos chunk_pos(const int32_t* se, int ci) {
  ChunkPos p;
  p.seq_start = se[SQ_START];
  p.t0 = p.seq_start + kC * ci;
  p.len = min(kC, se[SQ_LEN] - kC * ci);
  p.slot = se[SQ_SLOT];
  p.pos0 = static_cast<uint32_t>(se[SQ_POS0]);
  p.init = (se[SQ_FLAGS] & SQF_INIT) != 0;
  return p;
}

// Where chunk `chunk` of the call lies: its sequence is the last s whose
// first chunk is <= chunk.
__device__ __forceinline__ ChunkPos item_pos(const PrefillArgs& A, const PrefillLayout& Lay, int chunk) {
  const int32_t* stab = ws_ptr<int32_t>(A.workspace, Lay.seq_tab);
  int lo = 0, hi_s = A.n_seqs - 1;
  while (lo < hi_s) {
    const int mid = (lo + hi_s + 1) >> 1;
    if (stab[8 * mid + SQ_FIRST] <= chunk) lo = mid; else hi_s = mid - 1;
  }
  const int32_t* se = stab + 8 * lo;
  return chunk_pos(se, chunk - se[SQ_FIRST]);
}

// Conv item `item` of k-head kh: item = (2 channels, 16 tokens), the q | k
// items (4 D of them) first, then the v items of the k-head's G v-heads.
// Returns the first channel; tq = the item's first token within the chunk.
template <int D>
__device__ __forceinline__ int conv_item_c0(int item, int kh, int Hk, int G, int& tq) {
  constexpr int NQK = 4 * D;
  if (item < NQK) {
    const int q = item / D, cc0 = 2 * (item % D);
    tq = 16 * q;
    return cc0 < D ? kh * D + cc0 : Hk * D + kh * D + (cc0 - D);
  }
  const int i2 = item - NQK;
  tq = 16 * (i2 / (G * D / 2));
  return 2 * Hk * D + kh * G * D + 2 * (i2 % (G * D / 2));
}

// The conv inputs of a later item (chunk, kh) requested into the L2, so that
// its conv finds them there: one 4-byte load per 64-byte line of the rows it
// reads (its q, k and v channels, tokens t0 - 3 .. t0 + len - 1 within the
// sequence), straight into a scratch LDS slot of the wave (no registers
// held), by threads t, t + nthr, ...
template <int D, bool BF16>
__device__ void prefetch_item_rows(const PrefillArgs& A, const PrefillLayout& Lay, int chunk, int kh, int t,
                                   int nthr, void* lds_slot) {
  using E = typename Pk<BF16>::E;
  constexpr int EPL64 = 64 / static_cast<int>(sizeof(E));  // channels per 64-byte line
  const ChunkPos cp = item_pos(A, Lay, chunk);
  const int G = A.Hv / A.Hk;
  const int lq = (D + EPL64 - 1) / EPL64, lv = (G * D + EPL64 - 1) / EPL64, per_row = 2 * lq + lv;
  const int r0 = max(cp.t0 - 3, cp.seq_start), nrow = cp.t0 + cp.len - r0;
  const E* x = static_cast<const E*>(A.x);
  for (int i = t; i < nrow * per_row; i += nthr) {
    const int row = r0 + i / per_row, l = i % per_row;
    const int ch = l < lq ? kh * D + l * EPL64
                          : (l < 2 * lq ? A.Hk * D + kh * D + (l - lq) * EPL64
                                        : 2 * A.Hk * D + kh * G * D + (l - 2 * lq) * EPL64);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(x + static_cast<size_t>(row) * A.C + ch),
                                     (__attribute__((address_space(3))) void*)(lds_slot), 4, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// producer: one (chunk, k-head) item
// ---------------------------------------------------------------------------
// LDS of the producer, by lifetime:
//   R0: conv outputs of q | k (fp32), then L -> T of NH heads and Q K^T
//   R1: k (hi, lo for bf16) and q as A tiles
//   AM: K K^T;  MISC: per-token gate tables and norm factors
template <int D, bool BF16>
struct ProdSmem {
  using Gm = Geo<D, BF16>;
  static constexpr int NH = BF16 ? 3 : 1;            // v-heads per inverse group
  static constexpr int QK_LD = 2 * D + 4;            // rows 16-byte aligned
  static constexpr int PK_Q = BF16 ? 2 : 1;          // index of the q tiles in R1
  static constexpr size_t LT1 = static_cast<size_t>(kC) * kLd * 4;
  static constexpr size_t R0A = static_cast<size_t>(kC) * QK_LD * 4;
  static constexpr size_t R0B = (NH + 1) * LT1;
  static constexpr size_t R0 = R0A > R0B ? R0A : R0B;
  static constexpr size_t R1 = (PK_Q + 1) * 4 * Gm::KSD * kTileBytes;
  static constexpr size_t AM = LT1;
  static constexpr size_t MISC = static_cast<size_t>(4 * kMaxGroup * kC + 2 * kC) * 4;
  static constexpr size_t BYTES = R0 + R1 + AM + MISC;
};

template <int D, bool BF16, int NCG>
struct SmemBytes {
  static constexpr size_t P = ProdSmem<D, BF16>::BYTES;
  static constexpr size_t Ch = Geo<D, BF16, NCG>::NBUF * Geo<D, BF16, NCG>::STAGE_BYTES;
  static constexpr size_t value = P > Ch ? P : Ch;
  static_assert(value <= 158 * 1024, "LDS plan exceeds the CU's LDS");
};

// The workgroup's next ticket is taken from tctr at the start and left in
// *next_ticket (LDS) half-way, as the item it names (ticket + t_off), so no
// round trip separates one item from the next, and the next item's conv
// inputs are requested while this one inverts.  Item i < n_tickets is
// (chunk i / nk, k-head kh_base + 8 (i % nk)).  With tctr null no ticket is
// taken and n_tickets is left there (an item done on its own).
template <int D, bool BF16, int KW, int NCG>
__device__ void produce(const PrefillArgs& A, const PrefillLayout& Lay, char* sb, int chunk, int kh,
                        int32_t* tctr, int* next_ticket, int nk, int n_tickets, int kh_base, int t_off) {
  using P = Pk<BF16>;
  using Gm = Geo<D, BF16>;
  using Sm = ProdSmem<D, BF16>;
  using Ch = Chain<BF16>;
  using Bop = typename Ch::Bop;
  using E = typename P::E;
  constexpr int KSD = Gm::KSD, KSC = Gm::KSC, SK = P::SK, EPL = P::EPL, NT = Gm::NT;
  constexpr int NH = Sm::NH, QK_LD = Sm::QK_LD, NTRI = Gm::NTRI;
  float* smem = reinterpret_cast<float*>(sb);
  float* qk = smem;                                        // [64][QK_LD] conv outputs of q | k
  float* Lt = smem;                                        // NH x [64][65]: L -> T
  float* QKm = smem + NH * kC * kLd;                       // [64][65] Q K^T
  uint4* pk = reinterpret_cast<uint4*>(sb + Sm::R0);       // k (hi, lo) and q as A tiles
  float* Am = reinterpret_cast<float*>(sb + Sm::R0 + Sm::R1);  // [64][65] K K^T
  float* gcum = Am + kC * kLd;                             // [8][64] G
  float* bet = gcum + kMaxGroup * kC;                      // [8][64] beta
  float* dkf = bet + kMaxGroup * kC;                       // [8][64] e^{G_last - G}
  float* egt = dkf + kMaxGroup * kC;                       // [8][64] e^G
  float* inv = egt + kMaxGroup * kC;                       // [2][64] q and k norm factors

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk;
  const int RS = Lay.ring_slots;
  int32_t* hdr = ws_ptr<int32_t>(A.workspace, Lay.hdr);
  int32_t nxt = n_tickets;
  if (tid == 0 && tctr != nullptr) nxt = atomicAdd(tctr, 1) + t_off;
  const ChunkPos cp = item_pos(A, Lay, chunk);
  const int t0 = cp.t0, len = cp.len;
  char* rb = static_cast<char*>(A.workspace) + Lay.ring +
             (static_cast<size_t>(chunk % RS) * Hk + kh) * Lay.item_bytes;
  auto rtile = [&](int t) { return rb + static_cast<size_t>(t) * kTileBytes + 16 * lane; };
  auto htile = [&](int hi, int t) { return rtile(Gm::HEAD0 + hi * Gm::HEAD_TILES + t); };

  // The ring slot is free once every chain workgroup of this k-head has staged
  // the chunk it held (RS chunks earlier).  One thread waits; the barrier
  // keeps every wave's stores to the slot behind that wait.  It comes after
  // the conv's first input rows are requested, so they arrive during it.
  // Lane i of wave 0 polls chain i's counter, so all of them are read in one
  // round trip.
  static_assert(kMaxGroup * NCG <= 64, "one lane per chain of the k-head");
  auto wait_slot = [&]() {
    if (chunk >= RS) {
      if (wave == 0 && lane < G * NCG) {
        const int32_t* consumed = ws_ptr<int32_t>(A.workspace, Lay.consumed);
        wait_at_least(consumed + (kh * G * NCG + lane) * kLine, chunk - RS + 1, hdr + HDR_ABORT, A.dev_err);
      }
      lds_barrier();
    }
  };

  // gate inputs of the v-head whose gates this wave computes (the last G
  // waves, one head each: they have the fewest conv items), requested before
  // the conv's inputs, so they arrive first
  static_assert(kMaxGroup <= kWaves, "one gate head per wave");
  const int ghi = kWaves - 1 - wave;
  E a_raw{}, b_raw{};
  if (ghi < G && lane < len) {
    const size_t i = static_cast<size_t>(t0 + lane) * Hv + kh * G + ghi;
    a_raw = static_cast<const E*>(A.a)[i];
    b_raw = static_cast<const E*>(A.b)[i];
  }

  // ---- gates: one wave per v-head, lane = token, fixed-order inclusive scan;
  // run while the conv's inputs are on their way ----
  auto compute_gates = [&]() {
    if (ghi < G) {
      const int hi = ghi;
      float g = 0.f, bb = 0.f;
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
      gcum[hi * kC + lane] = g;
      bet[hi * kC + lane] = bb;
      dkf[hi * kC + lane] = __expf(glast - g);
      egt[hi * kC + lane] = __expf(g);
    }
  };

  // ---- conv + SiLU: item = (2 channels, 16 tokens); the q | k items first
  // (outputs to LDS), then the v items of the group's heads (V straight to the
  // ring in accumulator layout).  A thread takes items tid, tid + kThreads,
  // ...  With fp32 inputs the input rows of two of its items are requested
  // together before either is used; bf16 inputs come from the L2 (the
  // previous item requested them there), and one round at a time measured
  // faster, with fewer registers held. ----
  {
    constexpr int NQK = 4 * D;             // 2 D channels / 2 per item x 4 quarters
    constexpr int NB = BF16 ? 1 : 2;       // rounds whose loads are in flight together
    const int n_items = NQK + 2 * G * D;   // + G D v channels / 2 x 4 quarters
    auto item_c0 = [&](int item, int& tq) { return conv_item_c0<D>(item, kh, Hk, G, tq); };
    for (int base = 0; base < n_items; base += NB * kThreads) {
      Rows<BF16> raw[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int item = base + k * kThreads + tid;
        if (item < n_items) {
          int tq;
          const int c0 = item_c0(item, tq);
          load_rows<BF16, KW>(A, c0, tq, cp, raw[k]);
        }
      }
      if (base == 0) {
        wait_slot();  // before the first ring store
        compute_gates();
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int item = base + k * kThreads + tid;
        if (item >= n_items) continue;
        int tq;
        const int c0 = item_c0(item, tq);
        float y[2][16];
        conv_rows<BF16, KW>(A, c0, tq, cp, raw[k], y);
        if (item < NQK) {
          const int cc0 = 2 * (item % D);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            *reinterpret_cast<float2*>(qk + (tq + r) * QK_LD + cc0) = make_float2(y[0][r], y[1][r]);
        } else {
          const int i2 = item - NQK;
          const int q = tq / 16, vc = 2 * (i2 % (G * D / 2));   // v channel within the group
          const int hi = vc / D, dv0 = vc % D;
          E* vb = reinterpret_cast<E*>(htile(hi, Gm::HV) - 16 * lane);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            E* dst = vb + (((dv0 >> 4) * 4 + q) * 64 + g4 * 16 + (dv0 & 15)) * 4;
            if constexpr (BF16) {
              *reinterpret_cast<uint4*>(dst) =
                  make_uint4(pack2_bf16(y[0][4 * g4], y[0][4 * g4 + 1]), pack2_bf16(y[0][4 * g4 + 2], y[0][4 * g4 + 3]),
                             pack2_bf16(y[1][4 * g4], y[1][4 * g4 + 1]), pack2_bf16(y[1][4 * g4 + 2], y[1][4 * g4 + 3]));
            } else {
              *reinterpret_cast<float4*>(dst) = make_float4(y[0][4 * g4], y[0][4 * g4 + 1], y[0][4 * g4 + 2], y[0][4 * g4 + 3]);
              *reinterpret_cast<float4*>(dst + 4) = make_float4(y[1][4 * g4], y[1][4 * g4 + 1], y[1][4 * g4 + 2], y[1][4 * g4 + 3]);
            }
          }
        }
      }
    }
  }

  lds_barrier();

  // ---- L2 norm factors of q and k per token: 8 lanes per token, fixed order ----
  {
    const bool norm = (A.flags & GDN_FLAG_L2NORM_QK) != 0;
    constexpr int PER = D / 8;
    const int r = wave * 8 + (lane >> 3), part = lane & 7;
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
    if (part == 0) {
      inv[r] = norm ? A.q_scale * (1.0f / sqrtf(sq + A.l2_eps)) : A.q_scale;
      inv[kC + r] = norm ? 1.0f / sqrtf(sk + A.l2_eps) : 1.0f;
    }
  }
  lds_barrier();
  auto pack = [&](const float (&v)[EPL]) { return pack_lane<BF16>([&](int e) { return v[e]; }); };

  // ---- packing: Q and K as A tiles (rows token, k = d) to the ring, K (hi, lo)
  // and Q into LDS; for fp32 inputs K^T as A (rows d, k = token) to the ring;
  // gate tiles.
  // Every thread reads all the conv outputs and norm factors of its units
  // (both kinds, every round) before it packs any. ----
  {
    // (K^T tiles only for fp32 inputs: the bf16 chain reads K^T from the K
    // tiles with transposing LDS reads)
    constexpr int NQA = 4 * KSD * 64, NKT = BF16 ? 0 : NT * KSC * 64;
    constexpr int RQA = (NQA + kThreads - 1) / kThreads, RKT = BF16 ? 1 : (NKT + kThreads - 1) / kThreads;
    float kv[RQA][EPL], qv[RQA][EPL], kq_inv[RQA][2], kt[RKT][EPL], kt_inv[RKT][EPL];
#pragma unroll
    for (int rr = 0; rr < RQA; ++rr) {
      const int u = tid + rr * kThreads;
      const int tile = (u >> 6) % (4 * KSD), ln = u & 63;
      const int mt = tile / KSD, ks = tile % KSD;
      const int row = 16 * mt + (ln & 15), g = ln >> 4;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int k = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
        kv[rr][e] = k < D ? qk[row * QK_LD + D + k] : 0.f;
        qv[rr][e] = k < D ? qk[row * QK_LD + k] : 0.f;
      }
      kq_inv[rr][0] = inv[row];
      kq_inv[rr][1] = inv[kC + row];
    }
#pragma unroll
    for (int rr = 0; rr < (BF16 ? 0 : RKT); ++rr) {
      const int u = tid + rr * kThreads;
      const int tile = (u >> 6) % (NT * KSC), ln = u & 63;
      const int dt = tile / KSC, ks = tile % KSC;
      const int dk = 16 * dt + (ln & 15), g = ln >> 4;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int r = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
        kt[rr][e] = qk[r * QK_LD + D + dk];
        kt_inv[rr][e] = inv[kC + r];
      }
    }
#pragma unroll
    for (int rr = 0; rr < RQA; ++rr) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        settle(kv[rr][e]);
        settle(qv[rr][e]);
      }
      settle(kq_inv[rr][0]);
      settle(kq_inv[rr][1]);
    }
#pragma unroll
    for (int rr = 0; rr < (BF16 ? 0 : RKT); ++rr)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        settle(kt[rr][e]);
        settle(kt_inv[rr][e]);
      }
#pragma unroll
    for (int rr = 0; rr < RQA; ++rr) {
      const int u = tid + rr * kThreads;
      if (u >= NQA) continue;
      const int tile = u >> 6, ln = u & 63;
      float kn_[EPL], qn_[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kn_[e] = kv[rr][e] * kq_inv[rr][1];
        qn_[e] = qv[rr][e] * kq_inv[rr][0];
      }
      const uint4 qw = pack(qn_), kw = pack(kn_);
      *reinterpret_cast<uint4*>(rb + static_cast<size_t>(Gm::QA + tile) * kTileBytes + 16 * ln) = qw;
      *reinterpret_cast<uint4*>(rb + static_cast<size_t>(Gm::KA + tile) * kTileBytes + 16 * ln) = kw;
      pk[(Sm::PK_Q * 4 * KSD + tile) * 64 + ln] = qw;
      pk[tile * 64 + ln] = kw;
      if constexpr (BF16) {
        float lo_[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) lo_[e] = kn_[e] - bf16_bits_to_f32(f32_to_bf16_bits(kn_[e]));
        pk[(4 * KSD + tile) * 64 + ln] = pack(lo_);
      }
    }
#pragma unroll
    for (int rr = 0; rr < (BF16 ? 0 : RKT); ++rr) {
      const int u = tid + rr * kThreads;
      if (u >= NKT) continue;
      const int tile = u >> 6, ln = u & 63;
      float kn_[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) kn_[e] = kt[rr][e] * kt_inv[rr][e];
      *reinterpret_cast<uint4*>(rb + static_cast<size_t>(Gm::KT + tile) * kTileBytes + 16 * ln) = pack(kn_);
    }
  }
  for (int u = tid; u < G * 64; u += kThreads) {
    const int hi = u >> 6, ln = u & 63;
    float* gt = reinterpret_cast<float*>(rb + static_cast<size_t>(Gm::HEAD0 + hi * Gm::HEAD_TILES + Gm::HG) * kTileBytes);
    gt[Gm::G_EG + ln] = egt[hi * kC + ln];
    gt[Gm::G_D + ln] = dkf[hi * kC + ln];
    gt[Gm::G_G + ln] = gcum[hi * kC + ln];
    gt[Gm::G_EGL + ln] = __expf(gcum[hi * kC + kC - 1]);
  }
  lds_barrier();

  // ---- K K^T and Q K^T, lower 16x16 tiles (ti >= tj), into LDS (fp32): one
  // task per tile.  K K^T feeds the inverse: hi*hi + hi*lo + lo*hi for about
  // fp32 accuracy, in three independent accumulators. ----
  const uint4* kh_t = pk;
  const uint4* kl_t = pk + 4 * KSD * 64;
  const uint4* q_t = pk + Sm::PK_Q * 4 * KSD * 64;
  for (int task = wave; task < 10; task += kWaves) {
    int t = task, ti = 0;
    while (t > ti) { t -= ti + 1; ++ti; }
    const int tj = t;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, acc1 = acc, acc2 = acc, accq = acc;
    uint4 ah[KSD], bh[KSD], al[KSD], bl[KSD], qa[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      ah[ks] = kh_t[(ti * KSD + ks) * 64 + lane];
      bh[ks] = kh_t[(tj * KSD + ks) * 64 + lane];
      qa[ks] = q_t[(ti * KSD + ks) * 64 + lane];
      if constexpr (BF16) {
        al[ks] = kl_t[(ti * KSD + ks) * 64 + lane];
        bl[ks] = kl_t[(tj * KSD + ks) * 64 + lane];
      }
    }
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      acc = Ch::step(ah[ks], __builtin_bit_cast(Bop, bh[ks]), acc);
      accq = Ch::step(qa[ks], __builtin_bit_cast(Bop, bh[ks]), accq);
      if constexpr (BF16) {
        acc1 = Ch::step(ah[ks], __builtin_bit_cast(Bop, bl[ks]), acc1);
        acc2 = Ch::step(al[ks], __builtin_bit_cast(Bop, bh[ks]), acc2);
      }
    }
    if constexpr (BF16) acc = acc + (acc1 + acc2);
    const int g = lane >> 4, j = 16 * tj + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Am[(16 * ti + 4 * g + i) * kLd + j] = acc[i];
      QKm[(16 * ti + 4 * g + i) * kLd + j] = accq[i];
    }
  }
  if (tid == 0) *next_ticket = nxt;
  lds_barrier();

  // The waves without work in the next phase (first_wave and up) request the
  // next item's conv inputs into the L2; their LDS slots lie in the packed
  // tiles, which are no longer read.
  auto prefetch_next = [&](int first_wave) {
    if (wave >= first_wave) {
      const int t = *next_ticket;
      if (t < n_tickets)
        prefetch_item_rows<D, BF16>(A, Lay, t / nk, kh_base + kXcd * (t % nk), tid - first_wave * 64,
                                    (kWaves - first_wave) * 64, reinterpret_cast<char*>(pk) + wave * 256);
    }
  };
  if constexpr (NTRI < kWaves) prefetch_next(NTRI);

  // ---- per (packed P tile, lane): row r, EPL columns j; the decay
  // e^{G_r - G_j} of each v-head serves both P_rj = e^{G_r - G_j} (q_r . k_j),
  // j <= r (ring, every v-head) and L_rj = beta_r e^{G_r - G_j} (k_r . k_j),
  // j < r (LDS, the first inverse group).  The tiles cover every j < r. ----
  for (int u = tid; u < NTRI * 64; u += kThreads) {
    const int pt = u >> 6, ln = u & 63;
    int mt, ks;
    TriTiles<BF16>::at(pt, mt, ks);
    const int r = 16 * mt + (ln & 15), g = ln >> 4;
    float kk[EPL], qq[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int j = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
      kk[e] = Am[r * kLd + j];  // any value at j >= r; masked below
      qq[e] = QKm[r * kLd + j];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      settle(kk[e]);
      settle(qq[e]);
    }
    for (int hi = 0; hi < G; ++hi) {
      const float* gc = gcum + hi * kC;
      float gr = gc[r], br = bet[hi * kC + r], gj[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) gj[e] = gc[ks * SK + (e >> 2) * 16 + 4 * g + (e & 3)];
      settle(gr);
      settle(br);
#pragma unroll
      for (int e = 0; e < EPL; ++e) settle(gj[e]);
      float pv[EPL];
      float* Lr = Lt + hi * kC * kLd + r * kLd;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int j = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
        const float d = __expf(j <= r ? gr - gj[e] : 0.f);
        const float pvv = d * qq[e];
        pv[e] = j <= r ? pvv : 0.f;
        if (hi < NH) {
          const float lv = br * d * kk[e];
          Lr[j] = j < r ? lv : 0.f;
        }
      }
      *reinterpret_cast<uint4*>(rb + static_cast<size_t>(Gm::HEAD0 + hi * Gm::HEAD_TILES + Gm::HP + pt) * kTileBytes +
                                16 * ln) = pack(pv);
    }
  }
  // LDS writes complete, then the barrier; not lds_barrier(), whose fence
  // would also wait for the prefetch's loads (they write LDS).  Nothing reads
  // their scratch slots, and every wave waits for them before publishing.
  lds_sync();

  if constexpr (NTRI >= kWaves) prefetch_next(min(NH, G));

  // ---- per group of NH v-heads: L, T = (I + L)^{-1}, then T diag(beta) ----
  for (int hg0 = 0; hg0 < G; hg0 += NH) {
    const int nh = min(NH, G - hg0);
    if (hg0 > 0) {  // later groups: L of this group from K K^T in LDS
      for (int e = tid; e < nh * kC * kC; e += kThreads) {
        const int i = e / (kC * kC), r = (e / kC) % kC, j = e % kC;
        const float* gc = gcum + (hg0 + i) * kC;
        float br = bet[(hg0 + i) * kC + r], grv = gc[r], gjv = gc[j], kk = Am[r * kLd + j];
        settle(br);
        settle(grv);
        settle(gjv);
        settle(kk);
        const float v = br * __expf(j < r ? grv - gjv : 0.f) * kk;
        Lt[i * kC * kLd + r * kLd + j] = j < r ? v : 0.f;
      }
      lds_barrier();
    }
    if (wave < nh) {
      invert_unit_lower64(Lt + wave * kC * kLd, lane);
    }
    lds_sync();  // as above
    // T diag(beta) as A tiles (rows r, k = j); only the tiles of the lower triangle
    for (int u = tid; u < nh * NTRI * 64; u += kThreads) {
      const int i = (u >> 6) / NTRI, t = (u >> 6) % NTRI, ln = u & 63;
      int mt, ks;
      TriTiles<BF16>::at(t, mt, ks);
      const int r = 16 * mt + (ln & 15), g = ln >> 4;
      const float* Ti = Lt + i * kC * kLd + r * kLd;
      const float* sc = bet + (hg0 + i) * kC;
      float tv[EPL], tl[EPL], bj[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int j = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
        tl[e] = Ti[j];  // any value above the diagonal; masked below
        bj[e] = sc[j];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        settle(tl[e]);
        settle(bj[e]);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int j = ks * SK + (e >> 2) * 16 + 4 * g + (e & 3);
        const float v = tl[e] * bj[e];
        tv[e] = j <= r ? v : 0.f;
      }
      *reinterpret_cast<uint4*>(rb + static_cast<size_t>(Gm::HEAD0 + (hg0 + i) * Gm::HEAD_TILES + Gm::HT + t) *
                                         kTileBytes + 16 * ln) = pack(tv);
    }
    lds_barrier();  // Lt is reused by the next group
  }

  // ---- publish (chunk, k-head): every wave's stores have reached the L2
  // (stores are acknowledged by the L2), then one flag store.  The readers are
  // on this XCD and read through the same L2. ----
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    int32_t* ready = ws_ptr<int32_t>(A.workspace, Lay.ready);
    __hip_atomic_store(ready + ((chunk % RS) * Hk + kh) * kLine, chunk + 1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// chain: one workgroup per v-head walks every sequence's chunks in order
// ---------------------------------------------------------------------------
// The chain of v-head h runs as NCG workgroups; workgroup cg owns the d_v
// tiles cg NTG .. cg NTG + NTG-1.  Its waves 0 .. NWC-1 compute: wave w holds
// the 16-row tiles cg NTG + CT w .. + CT-1 of d_v, i.e. columns of S^T, as NT
// accumulator tiles each.  Waves NWC .. 7 are helpers: for chunk c+1 while
// the compute waves work on chunk c, they wait for the producer's flag and
// copy the item's operand tiles from the L2 into LDS.  One workgroup barrier
// per chunk swaps the two LDS buffers (two barriers when the geometry leaves
// room for one buffer).
template <int D, bool BF16, int KW, bool CKPT, int NCG>
__device__ void chain_role(const PrefillArgs& A, const PrefillLayout& Lay, char* sb, int kh, int h, int cg) {
  using P = Pk<BF16>;
  using Gm = Geo<D, BF16, NCG>;
  using Ch = Chain<BF16>;
  using E = typename P::E;
  using Bop = typename Ch::Bop;
  constexpr int KSD = Gm::KSD, KSC = Gm::KSC, NT = Gm::NT, TPS = Gm::TPS, SK = P::SK;
  constexpr int CT = Gm::CT, NWC = Gm::NWC, NBUF = Gm::NBUF, NTRI = Gm::NTRI, NTG = Gm::NTG;
  constexpr int NHW = kWaves - NWC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int Hk = A.Hk, Hv = A.Hv, G = Hv / Hk, hi = h - kh * G, C = A.C;
  const int RS = Lay.ring_slots;
  const int S = A.n_seqs;
  const int32_t* stab = ws_ptr<int32_t>(A.workspace, Lay.seq_tab);
  int32_t* hdr = ws_ptr<int32_t>(A.workspace, Lay.hdr);
  auto buf = [&](int c) { return sb + static_cast<size_t>(NBUF == 2 ? (c & 1) : 0) * Gm::STAGE_BYTES; };
  // bf16: the staged K tiles hold lane L's 16 bytes in slot k_slot(L) (an
  // involution that keeps every 16 consecutive lanes together), so that the
  // 16 rows a transposing read of K^T takes in one 16-lane group (lanes
  // 4 g + m + 16 q, m, q < 4) lie in 16 different slots modulo 16, i.e. in
  // different LDS banks; the K products read slot k_slot(lane).
  auto k_slot = [](int L) { return L ^ (4 * ((L >> 4) & 3)); };

  if (wave >= NWC) {
    // ================= helper waves =================
    const int hw = wave - NWC;
    const int32_t* ready = ws_ptr<int32_t>(A.workspace, Lay.ready);
    int32_t* consumed = ws_ptr<int32_t>(A.workspace, Lay.consumed);
    const char* ringb = static_cast<const char*>(A.workspace) + Lay.ring;
    // The helper waves walk the same chunks as the compute waves (every valid
    // sequence's chunks in order).  Right after chunk c's barrier the buffer
    // of chunk c+1 is free (the compute waves are done with chunk c-1): the
    // helpers issue loads that write the item's tiles (the k-head's Q and K,
    // and K^T for fp32 inputs; this v-head's T diag(beta), P, gates and V of
    // the workgroup's columns) straight from the L2
    // into that buffer, so they land while chunk c is computed.  Before
    // chunk c+1's barrier each helper wave polls the producer's flag for
    // chunk c+2, which also waits for its own loads of chunk c+1.
    // The buffer refilled holds, in its V region, the output of the chunk
    // NBUF before (written there by the compute waves): each helper wave
    // requests the tiles outside the V region first, then reads the pieces of
    // that output that lie in the V tiles it overwrites itself, requests
    // those tiles and stores the pieces to o.
    constexpr int NCP = (Gm::STAGE_TILES + NHW - 1) / NHW;  // tiles loaded per helper wave
    constexpr int RW = CT * 16;            // d_v per compute wave's slice
    constexpr int VT0 = Gm::HEAD0 + Gm::HV;  // first tile of the V region
    constexpr int NVP = (Gm::STAGE_TILES - VT0 + NHW - 1) / NHW;  // V tiles per helper wave
    const int vt_first = VT0 + ((hw - VT0) % NHW + NHW) % NHW;     // first of them
    const size_t rowstride = static_cast<size_t>(Hv) * D;
    struct Pieces {
      uint4 v[NVP];
    };
    auto read_out = [&](int c) {
      Pieces ov;
#pragma unroll
      for (int q = 0; q < NVP; ++q) {
        const int t = min(vt_first + NHW * q, Gm::STAGE_TILES - 1);
        ov.v[q] = *reinterpret_cast<const uint4*>(buf(c) + static_cast<size_t>(t) * kTileBytes + 16 * lane);
      }
      wait_lds();  // read before this wave's loads overwrite the tiles
      return ov;
    };
    auto write_out = [&](int tok0, int clen, const Pieces& ov) {
      E* og = static_cast<E*>(A.o) + static_cast<size_t>(tok0) * rowstride + h * D + cg * NTG * 16;
#pragma unroll
      for (int q = 0; q < NVP; ++q) {
        const int t = vt_first + NHW * q;
        const int e = ((t - VT0) * kTileBytes + 16 * lane) / static_cast<int>(sizeof(E));
        const int w = e / (kC * RW), tok = (e % (kC * RW)) / RW, dv = w * RW + e % RW;
        if (t < Gm::STAGE_TILES && tok < clen)
          *reinterpret_cast<uint4*>(og + static_cast<size_t>(tok) * rowstride + dv) = ov.v[q];
      }
    };
    auto poll = [&](int c) {
      wait_at_least(ready + ((c % RS) * Hk + kh) * kLine, c + 1, hdr + HDR_ABORT, A.dev_err);
    };
    // chunk c's tiles, ring slot c % RS, into buf(c): the tiles before the V
    // region (v_part false) or those of the V region (true)
    auto fill = [&](int c, bool v_part) {
      const char* rb = ringb + (static_cast<size_t>(c % RS) * Hk + kh) * Lay.item_bytes;
      char* b = buf(c);
#pragma unroll
      for (int j = 0; j < NCP; ++j) {
        const int t = hw + j * NHW;
        const int src = t < Gm::HEAD0 ? t
                                      : Gm::HEAD0 + hi * Gm::HEAD_TILES + (t - Gm::HEAD0) + (t >= VT0 ? cg * Gm::NVG : 0);
        const bool kt_tile = BF16 && t >= Gm::KT && t < Gm::KT + NT * KSC;  // read from the K tiles instead
        const bool k_tile = BF16 && t >= Gm::KA && t < Gm::KA + 4 * KSD;
        if (t < Gm::STAGE_TILES && (t >= VT0) == v_part && !kt_tile)
          load_l2_to_lds(rb, static_cast<uint32_t>(src * kTileBytes + 16 * (k_tile ? k_slot(lane) : lane)),
                         b + static_cast<size_t>(t) * kTileBytes);
      }
    };
    // the walk as a cursor: token offset and length of the next chunk
    int cur_s = -1, cur_ci = 0, cur_nc = 0, cur_start = 0, cur_len = 0;
    auto advance = [&]() {
      ++cur_ci;
      while (cur_ci >= cur_nc && cur_s + 1 < S) {
        const int32_t* se = stab + 8 * ++cur_s;
        cur_ci = 0;
        cur_nc = (se[SQ_FLAGS] & SQF_VALID) ? se[SQ_NCHUNK] : 0;
        cur_start = se[SQ_START];
        cur_len = se[SQ_LEN];
      }
    };
    const int total = hdr[HDR_TOTAL];
    int prev_tok = 0, prev_len = 0;  // chunk c-1
    if (total > 0) {
      poll(0);
      fill(0, false);
      fill(0, true);
    }
    for (int c = 0; c < total; ++c) {
      advance();
      const int tok = cur_start + kC * cur_ci, len = min(kC, cur_len - kC * cur_ci);
      if (NBUF == 2 && c + 1 < total) poll(c + 1);
      wait_vm();   // this wave's loads of chunk c are in LDS
      lds_sync();  // chunk c staged
      if (hw == 0 && lane == 0)
        __hip_atomic_store(consumed + (h * NCG + cg) * kLine, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (NBUF == 2) {
        // the tiles outside the V region first: only the V region holds
        // output still to be read
        if (c + 1 < total) fill(c + 1, false);
        const Pieces ov = read_out(c - 1 < 0 ? 0 : c - 1);
        if (c + 1 < total) fill(c + 1, true);
        if (c >= 1) write_out(prev_tok, prev_len, ov);
      } else {
        lds_sync();  // the compute waves are done with the buffer
        const Pieces ov = read_out(c);
        if (c + 1 < total) {
          poll(c + 1);
          fill(c + 1, false);
          fill(c + 1, true);
        }
        write_out(tok, len, ov);
      }
      prev_tok = tok;
      prev_len = len;
    }
    lds_sync();  // the compute waves are done with the last chunk
    if (NBUF == 2 && total > 0) write_out(prev_tok, prev_len, read_out(total - 1));
    return;
  }

  // ================= compute waves =================
  const int wl0 = wave * CT;       // first d_v tile of this wave within the workgroup's (V region, O slice)
  const int dvt0 = cg * NTG + wl0;  // first 16-row tile of d_v
  int c = 0;
  for (int s = 0; s < S; ++s) {
    const int32_t* se = stab + 8 * s;
    if (!(se[SQ_FLAGS] & SQF_VALID)) continue;
    const int nc = se[SQ_NCHUNK], len = se[SQ_LEN], seq_start = se[SQ_START], slot = se[SQ_SLOT];
    const bool init = (se[SQ_FLAGS] & SQF_INIT) != 0;
    const uint32_t pos0 = static_cast<uint32_t>(se[SQ_POS0]);
    const int ckpt0 = se[SQ_CKPT0];
    float* Sg = A.state + (static_cast<size_t>(slot) * Hv + h) * D * D;

    // S^T slice: st[ct][i] holds S^T[16 i + 4 g + e][16 (dvt0 + ct) + col]
    f32x4_t st[CT][NT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (init) {
          const float4 v = *reinterpret_cast<const float4*>(Sg + static_cast<size_t>(16 * (dvt0 + ct) + col) * D + 16 * i + 4 * g);
          st[ct][i] = f32x4_t{v.x, v.y, v.z, v.w};
        } else {
          st[ct][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
    auto store_state = [&](float* dst, const f32x4_t (&sv)[CT][NT]) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < NT; ++i)
          *reinterpret_cast<float4*>(dst + static_cast<size_t>(16 * (dvt0 + ct) + col) * D + 16 * i + 4 * g) =
              make_float4(sv[ct][i][0], sv[ct][i][1], sv[ct][i][2], sv[ct][i][3]);
    };

    for (int ci = 0; ci < nc; ++ci, ++c) {
      lds_sync();  // chunk c staged
      const char* base = buf(c);
      const int clen = min(kC, len - kC * ci);
      const uint4* qa = reinterpret_cast<const uint4*>(base + Gm::QA * kTileBytes);
      const uint4* ka = reinterpret_cast<const uint4*>(base + Gm::KA * kTileBytes);
      const uint4* kt = reinterpret_cast<const uint4*>(base + Gm::KT * kTileBytes);
      const uint4* ta = reinterpret_cast<const uint4*>(base + (Gm::HEAD0 + Gm::HT) * kTileBytes);
      const uint4* pa = reinterpret_cast<const uint4*>(base + (Gm::HEAD0 + Gm::HP) * kTileBytes);
      const float* gt = reinterpret_cast<const float*>(base + (Gm::HEAD0 + Gm::HG) * kTileBytes);
      const E* vb = reinterpret_cast<const E*>(base + Gm::V_OFF);
      auto tile = [&](const uint4* arr, int t) { return arr[t * 64 + lane]; };
      // K^T as an A tile (rows d 16 dt.., k = tokens 32 ks..).  fp32: staged.
      // bf16: from the K tiles (rows token, k = d) with two transposing LDS
      // reads.  In each 16-lane group such a read hands lane j, as value m,
      // element j % 4 of the 8 bytes lane 4 m + j / 4 addresses; so lane
      // l = 16 g + s addresses, for read h, the four d values 16 dt + 4 (s % 4)
      // .. +3 of token 32 ks + 16 h + 4 g + s / 4, which the K tile of token
      // block 2 ks + h and d block dt / 2 holds in lane 4 g + s / 4 + 16 (s % 4),
      // elements 4 (dt % 2) .. +3 (LDS slot k_slot of that lane).  Lane l then
      // holds d = 16 dt + s and tokens 32 ks + 16 h + 4 g + m, the A layout.
      auto kt_tile = [&](int dt, int ks) -> uint4 {
        if constexpr (BF16) {
          typedef short v4i16 __attribute__((ext_vector_type(4)));
          const int kl = k_slot(4 * (lane >> 4) + ((lane & 15) >> 2) + 16 * (lane & 3));
          uint2 w[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const char* p = reinterpret_cast<const char*>(ka) +
                            static_cast<size_t>((2 * ks + h) * KSD + (dt >> 1)) * kTileBytes + 16 * kl + 8 * (dt & 1);
            w[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                 (__attribute__((address_space(3))) v4i16*)(p)));
          }
          return make_uint4(w[0].x, w[0].y, w[1].x, w[1].y);
        } else {
          return tile(kt, dt * KSC + ks);
        }
      };

      // The step is ordered so that VALU work independent of the MFMAs in
      // flight is issued while they run: Y = K S^T and O^T = S Q^T back to
      // back; Z = V - diag(e^G) Y (its B operands) and the state's decay under
      // the O^T products; U = T diag(beta) Z; O^T scaled by e^G under U; U as B
      // operands (plain and decayed); O^T += U^T P^T and the state update; the
      // output last.  Scheduling barriers keep that order and bound the live
      // registers.  Inside a product the operand tiles of contraction step
      // ks+1 are read from LDS while the MFMAs of step ks run, and every tile
      // read feeds all CT tiles.
      auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
      // S^T as B operands (and, read the other way, S as A operands), built
      // once for both products of the state
      Bop bS[CT][KSD];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int i0 = ks * TPS;
          bS[ct][ks] = Ch::bop(st[ct][i0], (TPS == 2 && i0 + 1 < NT) ? st[ct][(i0 + 1) % NT] : f32x4_t{0.f, 0.f, 0.f, 0.f});
        }
      auto gvec = [&](int off, int mt) {
        const float4 v = *reinterpret_cast<const float4*>(gt + off + 16 * mt + 4 * g);
        return f32x4_t{v.x, v.y, v.z, v.w};
      };
      // acc[ct][mt] += A(mt, ks) S^T(ks) over ks (TR: the transposed product,
      // acc[ct][mt] += S(ks) A(mt, ks)^T, rows d_v and columns token): the
      // A tiles of one ks read ahead
      auto times_S = [&](const uint4* arr, f32x4_t (&acc)[CT][4], auto tr, int ln) {
        constexpr bool TR = decltype(tr)::value;
        uint4 cur[4], nxt[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) cur[mt] = arr[(mt * KSD) * 64 + ln];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          if (ks + 1 < KSD) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) nxt[mt] = arr[(mt * KSD + ks + 1) * 64 + ln];
          }
          fence();
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              acc[ct][mt] = TR ? Ch::step_t(bS[ct][ks], cur[mt], acc[ct][mt]) : Ch::step(cur[mt], bS[ct][ks], acc[ct][mt]);
          fence();
          if (ks + 1 < KSD) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) cur[mt] = nxt[mt];
          }
        }
      };
      const float eGl = gt[Gm::G_EGL];
      // Y = K S^T (rows token) and O^T = S Q^T (tile (ct, mt): rows d_v
      // 16 (dvt0 + ct) + 4 g + e, column token 16 mt + col, so a lane holds
      // four consecutive d_v of one token)
      f32x4_t Y[CT][4], O[CT][4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          Y[ct][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          O[ct][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      times_S(ka, Y, std::false_type{}, BF16 ? k_slot(lane) : lane);
      // V and e^G, read under the O^T products
      using VRaw = typename std::conditional<BF16, uint2, float4>::type;
      VRaw vr[CT][4];
      f32x4_t egv[4];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          vr[ct][mt] = *reinterpret_cast<const VRaw*>(vb + (((wl0 + ct) * 4 + mt) * 64 + lane) * 4);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) egv[mt] = gvec(Gm::G_EG, mt);
      times_S(qa, O, std::true_type{}, lane);
      // Z = V - diag(e^G) Y as B operands of the T product
      Bop bZ[CT][KSC];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          f32x4_t v;
          if constexpr (BF16) {
            const uint2 r2 = vr[ct][mt];
            v = f32x4_t{__uint_as_float(r2.x << 16), __uint_as_float(r2.x & 0xffff0000u),
                        __uint_as_float(r2.y << 16), __uint_as_float(r2.y & 0xffff0000u)};
          } else {
            const float4 r4 = vr[ct][mt];
            v = f32x4_t{r4.x, r4.y, r4.z, r4.w};
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) Y[ct][mt][e] = fmaf(-egv[mt][e], Y[ct][mt][e], v[e]);
        }
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) bZ[ct][ks] = Ch::bop(Y[ct][ks * TPS], Y[ct][(ks * TPS + 1) % 4]);
      }
      // the state's decay (a checkpoint inside the chunk still needs S itself)
      if constexpr (!CKPT) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int i = 0; i < NT; ++i) st[ct][i] = st[ct][i] * eGl;
      }
      fence();
      // U = T diag(beta) Z
      f32x4_t U[CT][4];
      {
        uint4 tt[NTRI];
#pragma unroll
        for (int t = 0; t < NTRI; ++t) tt[t] = tile(ta, t);
        fence();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            f32x4_t u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
              if (ks * SK <= 16 * mt + 15) u = Ch::step(tt[TriTiles<BF16>::index(mt, ks)], bZ[ct][ks], u);
            U[ct][mt] = u;
          }
      }
      // O^T scaled by e^G (per token column) while U runs; the P and K^T tiles read
      uint4 pt[NTRI];
#pragma unroll
      for (int t = 0; t < NTRI; ++t) pt[t] = tile(pa, t);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float e = gt[Gm::G_EG + 16 * mt + col];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) O[ct][mt] = O[ct][mt] * e;
      }
      fence();
      // U as B operands: plain (for P U) and decayed by e^{G_last - G} (for the state)
      Bop bU[CT][KSC], bUd[CT][KSC];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4_t Ud[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Ud[mt] = U[ct][mt] * gvec(Gm::G_D, mt);
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) {
          bU[ct][ks] = Ch::bop(U[ct][ks * TPS], U[ct][(ks * TPS + 1) % 4]);
          bUd[ct][ks] = Ch::bop(Ud[ks * TPS], Ud[(ks * TPS + 1) % 4]);
        }
      }
      // K^T tiles for the state update (read after the checkpoints when
      // there are any, which take them from LDS themselves)
      uint4 ktt[NT][KSC];
      auto load_ktt = [&] {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks) ktt[i][ks] = kt_tile(i, ks);
      };
      if constexpr (!CKPT) load_ktt();
      fence();
      // O^T += U^T P^T
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          f32x4_t o = O[ct][mt];
#pragma unroll
          for (int ks = 0; ks < KSC; ++ks)
            if (ks * SK <= 16 * mt + 15) o = Ch::step_t(bU[ct][ks], pt[TriTiles<BF16>::index(mt, ks)], o);
          O[ct][mt] = o;
        }
      // O of this chunk into this wave's own slice of the V region (read only
      // by this wave, in the step's first products): row-major [64 tokens][CT
      // 16 d_v].  The helper waves store it to o before the buffer is refilled,
      // so that no store of this wave has to complete before its registers
      // are reused.
      auto write_o = [&] {
        E* ol = reinterpret_cast<E*>(const_cast<char*>(base) + Gm::V_OFF) + wl0 * 4 * 256;
        constexpr int RW = CT * 16;                // d_v of a token row in this slice
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            E* dst = ol + (16 * mt + col) * RW + 16 * ct + 4 * g;
            if constexpr (BF16) {
              *reinterpret_cast<uint2*>(dst) = make_uint2(pack2_bf16(O[ct][mt][0], O[ct][mt][1]),
                                                          pack2_bf16(O[ct][mt][2], O[ct][mt][3]));
            } else {
              *reinterpret_cast<float4*>(dst) = make_float4(O[ct][mt][0], O[ct][mt][1], O[ct][mt][2], O[ct][mt][3]);
            }
          }
      };
      if constexpr (CKPT) write_o();  // O is not kept live across the checkpoints
      // state checkpoints inside this chunk: p = m * every in (64 ci, 64 ci + clen);
      // the state after token r = p - 64 ci - 1 of the chunk is
      // e^{G_r} S + K^T diag(d^(r)) U.  One at the chunk's end is the updated state.
      if (CKPT && A.ckpt_every > 0) {
        const int every = A.ckpt_every;
        const int done0 = kC * ci;
        for (int m = done0 / every + 1; m * every < done0 + clen; ++m) {
          const int r = m * every - done0 - 1;
          const float Gr = gt[Gm::G_G + r];
          f32x4_t dr[4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const f32x4_t gj = gvec(Gm::G_G, mt);
            const int j0 = 16 * mt + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) dr[mt][e] = j0 + e <= r ? __expf(Gr - gj[e]) : 0.f;
          }
          const float eGr = __expf(Gr);
          float* cdst = A.ckpt + (static_cast<size_t>(ckpt0 + m - 1) * Hv + h) * D * D;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            Bop bR[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) bR[ks] = Ch::scaled(bU[ct][ks], dr[ks * TPS], dr[(ks * TPS + 1) % 4]);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
              f32x4_t a = st[ct][i] * eGr;
#pragma unroll
              for (int ks = 0; ks < KSC; ++ks) a = Ch::step(kt_tile(i, ks), bR[ks], a);
              *reinterpret_cast<float4*>(cdst + static_cast<size_t>(16 * (dvt0 + ct) + col) * D + 16 * i + 4 * g) =
                  make_float4(a[0], a[1], a[2], a[3]);
            }
          }
        }
      }

      if constexpr (CKPT) {
        load_ktt();
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int i = 0; i < NT; ++i) st[ct][i] = st[ct][i] * eGl;
      }
      // S^T <- e^{G_last} S^T + K^T diag(e^{G_last - G}) U: all NT x CT
      // accumulators advance one contraction step at a time, so NT * CT
      // independent MFMAs are in flight between dependent ones
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) st[ct][i] = Ch::step(ktt[i][ks], bUd[ct][ks], st[ct][i]);
      fence();
      if constexpr (!CKPT) write_o();
      if (CKPT && A.ckpt_every > 0) {
        const int done = kC * ci + clen;
        if (done % A.ckpt_every == 0)
          store_state(A.ckpt + (static_cast<size_t>(ckpt0 + done / A.ckpt_every - 1) * Hv + h) * D * D, st);
      }

      if (NBUF == 1) lds_sync();  // buffer free for the next chunk
    }

    // ---- final state back to the slot ----
    store_state(Sg, st);
    // ---- conv history: the last W-1 inputs go to ring rows pos_end-1 .. pos_end-W+1
    // (by the first column group of each head) ----
    if (A.W > 0 && cg == 0) {
      const int W = A.W, R = A.R;
      const uint32_t pos_end = (init ? pos0 : 0u) + static_cast<uint32_t>(len);
      float* ring = A.conv_state + static_cast<size_t>(slot) * R * C;
      auto put = [&](int ch) {
        for (int i = 1; i < W; ++i) {
          const int rel = len - i;
          float* dst = ring + static_cast<size_t>(ring_row(pos_end - i, R)) * C + ch;
          if (rel >= 0) *dst = load_in<BF16>(A.x, static_cast<size_t>(seq_start + rel) * C + ch);
          else if (!init) *dst = 0.f;
        }
      };
      // the v channels of this head, and the q | k channels of the k-head (first v-head of the group)
      for (int cc = tid; cc < (hi == 0 ? 3 : 1) * D; cc += NWC * 64)
        put(cc < D ? 2 * Hk * D + h * D + cc : (cc < 2 * D ? kh * D + (cc - D) : Hk * D + kh * D + (cc - 2 * D)));
      if (A.last_seg && kh == A.kh_lo && hi == 0 && tid == 0)
        A.conv_pos[slot * kPosStride] = static_cast<int32_t>(pos_end << kPosShift);
    }
  }
  lds_sync();  // every chunk's O in LDS: the helpers store the last ones
}

// ---------------------------------------------------------------------------
// the fused launch: roles by per-XCD ticket
// ---------------------------------------------------------------------------
// CKPT: the variant that also writes state checkpoints (its chain keeps more
// values live; the plain prefill does not carry them).
template <int D, bool BF16, int KW, bool CKPT>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs A, PrefillLayout L) {
  constexpr int NCG = ncg_of<D, BF16>();
  __shared__ __attribute__((aligned(1024))) char smem[SmemBytes<D, BF16, NCG>::value];
  __shared__ int s_tk[2];
  const int tid = threadIdx.x;
  const int G = A.Hv / A.Hk;
  int32_t* ctr = ws_ptr<int32_t>(A.workspace, L.ctr) + static_cast<size_t>(A.seg) * kCtrLines * kLine;
  if (tid == 0) {
    const int x = xcc_id();
    s_tk[0] = x;
    s_tk[1] = atomicAdd(ctr + x * kLine, 1);
  }
  __syncthreads();
  const int xcc = s_tk[0], ticket = s_tk[1];
  // k-heads of this XCD in this launch: kh_lo + xcc + 8 j
  const int span = A.kh_hi - A.kh_lo;
  const int nk = span > xcc ? (span - xcc + kXcd - 1) / kXcd : 0;
  const int n_chain = nk * G * NCG;  // chains of this XCD: (k-head, v-head, column group)
  const int total = ws_ptr<int32_t>(A.workspace, L.hdr)[HDR_TOTAL];
  int chain_done = 0, items_done = 0;
  // Items of this XCD in chunk order.  A chain has nothing to do until chunk 0
  // is ready, so chain workgroup r first produces item r; the other
  // workgroups take items n_chain and up by ticket.  Item r < nk G NCG lies in
  // chunk r / nk < G NCG <= the ring depth (or the call has fewer chunks than
  // slots), so it never waits for a ring slot, which would need every chain of
  // its k-head, this one included, to have staged an earlier chunk.
  static_assert(kMaxGroup * NCG <= kRingSlots, "a chain's own item lies below the ring depth");
  const int n_items = total * nk;
  const bool is_chain = ticket < n_chain;
  int32_t* tctr = ctr + (kXcd + xcc) * kLine;
  if (nk > 0) {
    __syncthreads();  // s_tk is free
    if (tid == 0 && !is_chain) s_tk[1] = atomicAdd(tctr, 1) + n_chain;
    __syncthreads();
    for (int it = is_chain ? ticket : s_tk[1]; it < n_items; it = s_tk[1]) {
      produce<D, BF16, KW, NCG>(A, L, smem, it / nk, A.kh_lo + xcc + kXcd * (it % nk), is_chain ? nullptr : tctr,
                                &s_tk[1], nk, n_items, A.kh_lo + xcc, n_chain);
      ++items_done;
      if (is_chain) break;
    }
  }
  if (is_chain) {
    const int kh = A.kh_lo + xcc + kXcd * (ticket / (G * NCG));
    const int r = ticket % (G * NCG);
    chain_role<D, BF16, KW, CKPT, NCG>(A, L, smem, kh, kh * G + r / NCG, r % NCG);
    chain_done = 1;
  }
  // Last workgroup out: every chain role and every item must have been done.
  __syncthreads();
  if (tid == 0) {
    const unsigned long long add = (1ull << 48) | (static_cast<unsigned long long>(chain_done) << 32) |
                                   static_cast<unsigned long long>(items_done);
    const unsigned long long old =
        atomicAdd(reinterpret_cast<unsigned long long*>(ctr + 2 * kXcd * kLine), add);
    if ((old >> 48) == gridDim.x - 1) {
      const unsigned long long all = old + add;
      const unsigned long long want_chain = static_cast<unsigned long long>(span) * G * NCG;
      const unsigned long long want_items = static_cast<unsigned long long>(total) * span;
      if (((all >> 32) & 0xffffull) != want_chain || (all & 0xffffffffull) != want_items)
        report_error(A.dev_err, GDN_DEV_INCOMPLETE);
    }
  }
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------
template <int D, bool BF16>
static int launch_prefill_t(const PrefillArgs& a0, hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const PrefillLayout L = layout_t<D, BF16>(a0.Hk, a0.Hv, a0.n_tokens, a0.n_seqs);
  const int ncg = ncg_of<D, BF16>();
  const int n_launch = launches(a0.Hk, a0.Hv, ncg);
  const int per = heads_per_launch(a0.Hk, a0.Hv, ncg);
  if (ev_start != nullptr || ev_stop != nullptr) {
    // an event recorded under capture would not time anything: refuse
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t ce = hipStreamIsCapturing(st, &cs);
    if (ce != hipSuccess) return static_cast<int>(ce);
    if (cs != hipStreamCaptureStatusNone) return static_cast<int>(hipErrorStreamCaptureUnsupported);
  }
  // `start` is the plan kernel's completion, where the main kernel begins (a
  // launch's start event can be stamped before the previous kernel is done)
  if (ev_start != nullptr)
    hipExtLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, nullptr, ev_start, 0, a0, L, n_launch);
  else
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, a0, L, n_launch);
  int e = static_cast<int>(hipGetLastError());
  if (e) return e;
  auto fn = a0.ckpt_every > 0 ? (a0.W == 4 ? &prefill_kernel<D, BF16, 4, true> : &prefill_kernel<D, BF16, 0, true>)
                              : (a0.W == 4 ? &prefill_kernel<D, BF16, 4, false> : &prefill_kernel<D, BF16, 0, false>);
  for (int seg = 0; seg < n_launch; ++seg) {
    PrefillArgs a = a0;
    a.kh_lo = seg * per;
    a.kh_hi = a.kh_lo + per < a0.Hk ? a.kh_lo + per : a0.Hk;
    a.seg = seg;
    a.last_seg = seg == n_launch - 1;
    hipEvent_t ee = seg == n_launch - 1 ? ev_stop : nullptr;
    if (ee != nullptr)
      hipExtLaunchKernelGGL(fn, dim3(kXcd * kWgPerXcd), dim3(kThreads), 0, st, nullptr, ee, 0, a, L);
    else
      hipLaunchKernelGGL(fn, dim3(kXcd * kWgPerXcd), dim3(kThreads), 0, st, a, L);
    e = static_cast<int>(hipGetLastError());
    if (e) return e;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// The workspace of the prefill that allocates nothing: a static array, one per
// GPU, held until the process ends.  Host code uses only the device address
// looked up per GPU, never the array's name (a host-side stand-in).
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[GDN_PREFILL_STATIC_WORKSPACE_BYTES];

int prefill_static_workspace(void* stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return static_cast<int>(e);
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return static_cast<int>(e);
  }
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return static_cast<int>(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return static_cast<int>(e);
    if (p == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_prefill(const PrefillArgs& a, bool bf16, void* stream, void* ev_start, void* ev_stop) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
  switch (a.D) {
    case 16: return bf16 ? launch_prefill_t<16, true>(a, s, e0, e1) : launch_prefill_t<16, false>(a, s, e0, e1);
    case 32: return bf16 ? launch_prefill_t<32, true>(a, s, e0, e1) : launch_prefill_t<32, false>(a, s, e0, e1);
    case 64: return bf16 ? launch_prefill_t<64, true>(a, s, e0, e1) : launch_prefill_t<64, false>(a, s, e0, e1);
    case 128:
      if (bf16) return launch_prefill_t<128, true>(a, s, e0, e1);
      return static_cast<int>(hipErrorInvalidValue);  // refused by the API before any launch
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace gdn
