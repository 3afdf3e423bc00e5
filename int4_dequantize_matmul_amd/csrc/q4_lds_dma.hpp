// Staging helpers of the LDS-tiled kernels (gfx950): raw buffer resources,
// buffer loads that write LDS, and waits on the vector-memory count.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef __attribute__((address_space(3))) void lds_void;

// LDS address of a pointer into shared memory (the M0 operand of a load
// that writes LDS).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p));
}

// Raw buffer resource over bytes [p, p + bytes): loads past the end read 0,
// stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int bytes) {
  // raw buffer, bounds = bytes; dword 3 as for gfx9 raw buffers
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), bytes,
                                           0x00020000);
}

// s_waitcnt with only the vector-memory count constrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 16, "vmcnt range used here");
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  if constexpr (N == 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  if constexpr (N == 14) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
  if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  static_assert(N == 0 || (N >= 3 && N <= 8) || N == 10 || N == 12 || N == 14 || N == 16, "add the count");
}

// Buffer loads that write LDS: lane i's 16 bytes land at lds + 16 i (dma16);
// the 4-, 2- and 1-byte forms fill lane i's 4-byte slot at lds + 4 i (the
// value in its low bytes).  Written as assembly so that the compiler's own
// wait counting does not make every later LDS read wait for all of them;
// the kernels wait for them themselves (wait_vmcnt before each barrier).  M0
// carries the LDS address; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "m0");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "m0");
}
__device__ __forceinline__ void dma2(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "m0");
}
__device__ __forceinline__ void dma1(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ubyte %1, %2, %3 offen lds" ::"s"(lds), "v"(voff), "s"(r),
               "s"(soff)
               : "m0");
}
#pragma clang diagnostic pop

// Position of the 16-byte chunk c of a 128-byte LDS row r is c ^ swz8(r):
// every 8-lane phase of a read of one chunk from 8 consecutive rows then
// touches distinct banks.  It depends on r mod 16 only.
__device__ __forceinline__ int swz8(int r) {
  return ((r & 3) ^ ((r >> 2) & 1)) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
}

}  // namespace q4
