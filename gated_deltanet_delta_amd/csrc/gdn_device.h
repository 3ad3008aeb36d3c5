// Device helpers shared by the GDN kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

constexpr int kWave = 64;
constexpr int kPosShift = 16;  // conv_pos counts tokens in units of 1/65536
constexpr int kPosStride = GDN_POS_STRIDE;  // a slot's position is conv_pos[slot * kPosStride]

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 kept as its 16-bit pattern)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (the hardware v_cvt_pk_bf16_f32 of gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two values rounded to bf16 and packed (lo in bits 0-15): one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Element access for the two input/output dtypes: BF16 = true reads bf16 bits.
template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* p, size_t i, float v) {
  if constexpr (BF16) static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
  else static_cast<float*>(p)[i] = v;
}

// Four consecutive elements starting at element i (i multiple of 4).
template <bool BF16>
__device__ __forceinline__ float4 load_in4(const void* p, size_t i) {
  if constexpr (BF16) {
    const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  }
}

// ---------------------------------------------------------------------------
// Scalar laws: beta = sigmoid(b), g = log(alpha) = -softplus(a)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid_f(float x) { return 1.0f / (1.0f + expf(-x)); }
__device__ __forceinline__ float silu_f(float y) { return y * sigmoid_f(y); }

// ---------------------------------------------------------------------------
// Reductions inside groups of N consecutive lanes (N a power of two <= 64),
// always in the same butterfly order, so results are reproducible.
// ---------------------------------------------------------------------------
// Sum over aligned groups of N lanes, every lane of a group receiving the
// total (bitwise the same in every lane: each step adds a lane's value to its
// partner's, and the partners add the same two numbers).  Lane exchanges up to
// 16 apart use DPP (quad permutes and row mirrors), 16 and 32 use swizzle /
// bpermute.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "group size");
  if constexpr (N >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: partner lane ^ 1
  if constexpr (N >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: partner lane ^ 2
  if constexpr (N >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror: partner 7 - i within 8 lanes
  if constexpr (N >= 16) v += dpp_mov<0x140>(v); // row_mirror: partner 15 - i within 16 lanes
  if constexpr (N >= 32)                         // swizzle, and mask 31, xor mask 16: partner lane ^ 16
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if constexpr (N >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Workgroup barrier that orders LDS traffic only: global loads issued before
// it stay in flight (a full __syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// The same ordering written out: this wave's LDS operations complete
// (lgkmcnt), then the barrier; the compiler moves no memory access across
// it.  Nothing waits for the wave's global loads or stores (vmcnt).
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// SiLU and sigmoid with the hardware exp2 and reciprocal (about 2 ulp).  An
// argument so negative that 2^x underflows gives 1 + 0; so positive that it
// overflows gives rcp(inf) = 0.
__device__ __forceinline__ float sigmoid_fast(float y) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * y));
}
__device__ __forceinline__ float silu_fast(float y) {
  return y * sigmoid_fast(y);
}
// SiLU of y given s = -log2(e) y (a conv whose weights carry the factor):
// y / (1 + e^-y) = s / (-(1 + 2^s) / ln 2), one multiply fewer than silu_fast.
constexpr float kNegLog2e = -1.4426950408889634f;
__device__ __forceinline__ float silu_of_scaled(float s) {
  constexpr float kNegInvLn2 = -1.4426950408889634f;  // -1 / ln 2
  return s * __builtin_amdgcn_rcpf(fmaf(__builtin_amdgcn_exp2f(s), kNegInvLn2, kNegInvLn2));
}

// ---------------------------------------------------------------------------
// Device error word: the first code of a call wins.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void report_error(int32_t* dev_err, int32_t code) {
  if (dev_err) atomicCAS(dev_err, 0, code);
}

// Ring row of token position p (R a power of two).
__device__ __forceinline__ int ring_row(uint32_t p, int R) { return static_cast<int>(p & (R - 1)); }

// Non-temporal 16-byte store (state and snapshots are streamed, not reused).
__device__ __forceinline__ void store_nt4(float* p, f32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}
// Stores that write through this XCD's L2 to memory (cache policy sc1).
// Data a concurrently running kernel on another XCD reads goes out this way,
// so publishing it needs only the wave's own store counter (wait_stores), not
// a write-back of the whole L2.  They are buffer stores: `base` is the same
// in every lane of the wave (it becomes the buffer descriptor), `off` is the
// lane's byte offset from it.
constexpr int kStoreSc1 = 16;  // cache-policy operand of the buffer builtins: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wt_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  // raw buffer: stride 0, whole 2 GB range, 32-bit data format
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo),
                                           static_cast<short>(0), 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void store_wt(const void* base, uint32_t off, uint4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4{v.x, v.y, v.z, v.w}, wt_rsrc(base), off, 0, kStoreSc1);
}
__device__ __forceinline__ void store_wt(const void* base, uint32_t off, uint2 v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, wt_rsrc(base), off, 0, kStoreSc1);
}
__device__ __forceinline__ void store_wt(const void* base, uint32_t off, float4 v) {
  store_wt(base, off, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)));
}
__device__ __forceinline__ void store_wt(const void* base, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), wt_rsrc(base), off, 0, kStoreSc1);
}
// Wait until every vector memory access this wave issued has completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ f32x4_t load4(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}
// Makes x opaque to the compiler at this point: the reads that produced it
// are complete here and cannot be moved into a later conditional block, where
// each would be waited for on its own.
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)); }

// 16-byte non-temporal load: data read once, not kept in the caches.
__device__ __forceinline__ f32x4_t load_nt4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
}

}  // namespace gdn
