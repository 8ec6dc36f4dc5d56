// Device-side helpers shared by the gfx950 attention kernels: vector types,
// buffer-resource loads with hardware bounds checking, lane exchanges.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// A byte offset that is always past the end of a buffer resource: validation
// keeps every (batch, head) slice below 2^31 bytes, so loads at this offset
// return zeros without touching memory.
constexpr unsigned kOOB = 0x80000000u;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Raw buffer resource over [base, base + bytes).  Word 3 selects 32-bit data
// format with no swizzle, the setting for untyped loads on gfx9-class parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ unsigned buf_load4(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// Streaming loads (cache policy "nt", non-temporal) for data read exactly
// once, such as a KV cache during decode.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
}
__device__ __forceinline__ u32x2 buf_load8_nt(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
}

// Value held by lane (lane ^ 32): the other half of the wavefront.  One
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with x in both, the first result holds x's lower
// half in both halves and the second x's upper half, so lane l picks the
// second result when l < 32 and the first otherwise.  No LDS round trip.
__device__ __forceinline__ float swap_halves(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const bool low = (threadIdx.x & 32) == 0;
  return __builtin_bit_cast(float, low ? r[1] : r[0]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x on the FMA pipe instead of the transcendental unit (the FlashAttention
// interview canvas's v4 card moves part of the exponentials there).  Range
// reduction in the manner of Cody and Waite: x = n + f with n = rint(x) taken
// by the 1.5 * 2^23 rounding constant and f in [-1/2, 1/2]; 2^f by a degree-4
// polynomial whose coefficients were fitted here to the relative error of
// 2^f at Chebyshev nodes (maximum 2^-18.5 when evaluated in float32); n is
// added to the exponent field.  Valid for x <= 8 (the softmax's arguments stay
// below the lazy-max slack); arguments at or below -125 (masked scores are
// -inf) give exactly 0.
__device__ __forceinline__ float soft_exp2(float x) {
  constexpr float kRound = 0x1.8p23f;
  const float xc = fmaxf(x, -125.f);
  const float t = xc + kRound;  // 1.5 * 2^23 + rint(xc): rint(xc) in the low bits
  const float n = t - kRound;
  const float f = xc - n;
  float p = __builtin_fmaf(0x1.3997cap-7f, f, 0x1.ca1440p-5f);
  p = __builtin_fmaf(p, f, 0x1.ec06dap-3f);
  p = __builtin_fmaf(p, f, 0x1.62e0dcp-1f);
  p = __builtin_fmaf(p, f, 0x1.ffffe8p-1f);
  // (bits(t) << 23) = n << 23 modulo 2^32, since 1.5 * 2^23 has no bits below 2^9
  const unsigned bits = __builtin_bit_cast(unsigned, p) + (__builtin_bit_cast(unsigned, t) << 23);
  return x > -125.f ? __builtin_bit_cast(float, bits) : 0.f;
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).  Used after
// loads that must be complete on every path into a loop: it keeps the
// compiler's wait analysis at the loop head from re-waiting on them behind
// the loop's own prefetches.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The lane's index within its wavefront, computed where it is called: the
// opaque zero keeps the compiler from reusing an earlier value, which would
// then have to stay live through a register-bound loop (and be spilled, or
// crowd it) until here.  For rarely taken branches such as edge masks, and
// for epilogues.
__device__ __forceinline__ int fresh_lane_id() {
  int zero = 0;
  asm volatile("" : "+v"(zero));
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, static_cast<unsigned>(zero))));
}

// A DPP move within each row of 16 lanes.  Every pattern used here reads a
// lane inside the same row, so no lane is out of bounds; bound_ctrl set lets
// the move need no prior value in its destination.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// The value lane (l ^ X) holds, within each row of 16 lanes (X = 1, 2, 4, 8):
// one or two DPP moves on the vector ALU, where a width-16 shuffle would be
// an LDS permute.
template <int X>
__device__ __forceinline__ float row16_xor(float v) {
  static_assert(X == 1 || X == 2 || X == 4 || X == 8, "row16_xor: 1, 2, 4 or 8");
  if constexpr (X == 1) return dpp_mov<0xB1>(v);                  // quad_perm [1, 0, 3, 2]
  else if constexpr (X == 2) return dpp_mov<0x4E>(v);             // quad_perm [2, 3, 0, 1]
  else if constexpr (X == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(v));  // l ^ 7, then l ^ 3
  else return dpp_mov<0x141>(dpp_mov<0x140>(v));                  // l ^ 15, then l ^ 7
}

// True if pred holds in any lane of the wavefront (wave-uniform result).
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Marks x as produced at this point of the program: the empty volatile asm
// keeps the compiler from sinking the computation of x past it (for
// instance into a later loop iteration), so work dealt out between MFMAs
// stays where it was placed.  No instruction is emitted.
template <typename V> __device__ __forceinline__ void pin(V &x) { asm volatile("" : "+v"(x)); }

// f(integral_constant<int, I>) for I = 0 .. N-1, fully unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Sum / max of 16 floats as a balanced tree (short dependency chains).
__device__ __forceinline__ float tree_sum16(const float *x) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[i] + x[i + 8];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] += a[i + 4];
  return (a[0] + a[2]) + (a[1] + a[3]);
}

// Online-softmax lazy rescale threshold (log2 units): the running max moves
// only when a row's new max exceeds it by more than this, so probabilities
// stay below 2^kRescaleSlack and most tiles skip the O rescale entirely.
constexpr float kRescaleSlack = 8.0f;

}  // namespace fa
