// Device-side helpers shared by the libq4 kernels (gfx950 / CDNA4).
//
// Every kernel file is compiled with -ffp-contract=off: a multiply followed
// by an add stays two roundings unless a kernel asks for fmaf explicitly
// (the pages warn that letting the compiler fuse on some paths but not
// others changes bits; "Fused int4 and int8 dequantize-matmul in C",
// section 2.4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Planted mistakes for the mutation check of the GPU tests: a library built
// with -DQ4_MUTANT=n (n = 1..9) carries the n-th pitfall of "Fused int4 and
// int8 dequantize-matmul in C", section 5, in one kernel, and the test
// suite must fail on it.  The shipped library is built without it (0).
#ifndef Q4_MUTANT
#define Q4_MUTANT 0
#endif

namespace q4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> f32: the pattern is the top half of a binary32.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// IEEE half bit pattern -> f32, exactly (subnormal halves are normal f32).
__device__ __forceinline__ float f16_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// Finite f32 -> bf16 bit pattern, round to nearest, ties to even: add
// 0x7FFF plus the lowest kept bit, then truncate.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One activation code of the Q8 recipe: clamp(rint(v / scale), -127, 127)
// with the real quotient (never a product with a reciprocal) and ties to
// even; scale 0 gives 0.  Every kernel that quantizes activations calls
// this, so their codes agree bit for bit.
__device__ __forceinline__ float q8_code_f(float v, float scale) {
  if (scale == 0.0f) return 0.0f;
  float r = rintf(v / scale);
  return fminf(fmaxf(r, -127.0f), 127.0f);
}

__device__ __forceinline__ int8_t q8_code(float v, float scale) {
  return static_cast<int8_t>(static_cast<int>(q8_code_f(v, scale)));
}

// The Q8 code with the quotient v / s formed from r = RN(1/s) and one
// correction step (Markstein): y = RN(v r), e = v - s y exactly (fma), then
// RN(y + e r) is the correctly rounded quotient.  It needs s and the
// residual clear of the subnormal range, which holds whenever the row
// maximum is at least 2^-64 (then s >= 2^-71); q8_row_rcp gives r in that
// range and 0 otherwise (then the caller uses q8_code).  The identity is
// exercised on the host over the neighbourhoods of every rounding boundary.
__device__ __forceinline__ float q8_code_rcp_f(float v, float s, float r) {
  const float y = v * r;
  const float e = fmaf(-s, y, v);
  const float q = rintf(fmaf(e, r, y));
  return fminf(fmaxf(q, -127.0f), 127.0f);
}

__device__ __forceinline__ int8_t q8_code_rcp(float v, float s, float r) {
  return static_cast<int8_t>(static_cast<int>(q8_code_rcp_f(v, s, r)));
}

// RN(1 / s) for a row of maximum amax and scale s = RN(amax / 127), where
// q8_code_rcp is exact, else 0.
__device__ __forceinline__ float q8_row_rcp(float amax, float s) {
  return amax >= 0x1p-64f && amax <= 0x1p+100f ? 1.0f / s : 0.0f;
}

// Barrier that orders LDS only: waits for this wave's LDS traffic, then
// meets the other waves.  Outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 mfma_i8_16x16x64(uint4 a, uint4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// Byte selection from two dwords: result byte i = byte sel_i of {hi:lo}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Sum over each row of 16 lanes (WIDTH 16) or each half row (WIDTH 8) with
// DPP moves: pair swap, quad swap, half-row mirror, row mirror.  Every lane
// of the group ends with the same value (each step adds two equal-shaped
// partial sums in a commutative way).
template <int WIDTH>
__device__ __forceinline__ float dpp_row_sum_f32(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)); // row_half_mirror
  if constexpr (WIDTH == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)); // row_mirror
  return v;
}

// The value of lane l ^ 16 (xor16) or l ^ 32 (xor32), from the lane-swap
// instructions of this chip: no LDS round trip, unlike a shuffle.  Both
// operands of the swap are v: after v_permlane16_swap the pair holds, in
// every lane, the lane's own value and that of lane l ^ 16 (in some order);
// their sum or maximum is the same in either order.
__device__ __forceinline__ float add_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Integer forms (exact, so the order of the two addends does not matter).
__device__ __forceinline__ int add_xor16_i32(int v) {
  const auto p = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  return static_cast<int>(p[0]) + static_cast<int>(p[1]);
}
__device__ __forceinline__ int add_xor32_i32(int v) {
  const auto p = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  return static_cast<int>(p[0]) + static_cast<int>(p[1]);
}

// Maximum over the 64 lanes, in every lane.  The maximum is exact, so the
// order of the steps cannot change it.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  return max_xor32(max_xor16(v));
}

template <int WIDTH>
__device__ __forceinline__ int dpp_row_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  if constexpr (WIDTH == 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return v;
}

__device__ __forceinline__ uint4 load16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

}  // namespace q4
