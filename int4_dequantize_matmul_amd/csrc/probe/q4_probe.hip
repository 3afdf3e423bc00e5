// libq4_probe: ceilings for the benchmark (a streaming read, the int8
// matrix-core rate and the shader clock), measured on the running device.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../../include/q4_probe.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte chunks, four loads in flight per thread.
__global__ void probe_read_kernel(const u32x4 *__restrict__ p, uint64_t n16, uint32_t *__restrict__ sink) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // a store that depends on every thread's value keeps the loads alive;
  // thread 0 always writes, others only on one unlikely value
  if (threadIdx.x == 0 || acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256, 1) void probe_mfma_kernel(uint64_t *out, int iters) {
  const int lane = threadIdx.x & 63;
  i32x4 a = {lane, 1, 2, 3}, b = {3, lane, 5, 7};
  i32x16 acc[4];
  for (int j = 0; j < 4; ++j)
    for (int r = 0; r < 16; ++r) acc[j][r] = r + j;
  const uint64_t c0 = __builtin_amdgcn_s_memtime(), t0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime(), t1 = __builtin_amdgcn_s_memrealtime();
  int s = 0;
  for (int j = 0; j < 4; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (lane == 0) {
    out[2 * wave] = c1 - c0;
    out[2 * wave + 1] = (t1 - t0) + (s == 0x7FFFFFFF ? 1u : 0u);   // keeps the sums alive
  }
}

bool overlap(const void *a, uint64_t an, const void *b, uint64_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

}  // namespace

extern "C" q4_status q4_probe_read(const void *buf, size_t bytes, uint32_t *sink, int64_t blocks, int64_t threads,
                                   void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return Q4_EINVAL;
  if (blocks < 1 || blocks > 65535 || !(threads == 64 || threads == 128 || threads == 256 || threads == 512))
    return Q4_EINVAL;
  if (overlap(buf, bytes, sink, static_cast<uint64_t>(blocks) * 4)) return Q4_EINVAL;
  probe_read_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(static_cast<unsigned>(threads)), 0,
                      static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4 *>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? Q4_OK : Q4_EDEVICE;
}

extern "C" q4_status q4_probe_mfma_i8(uint64_t *out, int64_t blocks, int64_t iters, void *stream) {
  if (!out || blocks < 1 || blocks > 65535 || iters < 1 || iters > 1000000) return Q4_EINVAL;
  probe_mfma_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      out, static_cast<int>(iters));
  return hipGetLastError() == hipSuccess ? Q4_OK : Q4_EDEVICE;
}
