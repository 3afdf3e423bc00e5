// Activation quantizer and the zero fill.
//
// Canonical Q8 recipe, one activation row at a time (ftts_kernels module
// int8: quantize_row_q8, and the module head: activations quantized
// dynamically per row with the same recipe as the weights):
//   scale = max|x| / 127      (IEEE f32 division, correctly rounded)
//   q     = clamp(rint(x / scale), -127, 127), ties to even (v_rndne_f32)
// A row of zeros gives scale 0 and codes 0.  bf16 input is widened exactly.
//
// One workgroup of 256 threads owns one row: a max-reduction over the row,
// then the per-element quotient.  The quotient is the correctly rounded
// one, so the codes match a host quantizer bit for bit: formed from
// RN(1 / scale) with one correction step where that is exact (row maxima
// from 2^-64 to 2^100, q8_code_rcp), else by the division itself.  HBM
// traffic is one read of x (twice when the row does not stay in registers)
// and one write of xq.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max_f32(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

// Vector form: K % 8 == 0 and 16-byte aligned rows; each thread takes runs
// of 8 elements.  Rows of up to 8 * 256 elements stay in registers.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_rows_vec(const void *__restrict__ x, int64_t K,
                                                              int8_t *__restrict__ xq,
                                                              float *__restrict__ sx) {
  __shared__ float red[kThreads / 64];
  const int64_t m = blockIdx.x;
  const int64_t runs = K / 8;
  float v[8];
  float amax = 0.0f;
  const bool single = runs <= kThreads;
  auto load_run = [&](int64_t r, float *out) {
    if constexpr (BF16) {
      const uint4 d = load16(static_cast<const uint16_t *>(x) + m * K + r * 8);
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        out[2 * i + 1] = bf16_to_f32(w[i] >> 16);
      }
    } else {
      const float *p = static_cast<const float *>(x) + m * K + r * 8;
      const float4 a = *reinterpret_cast<const float4 *>(p);
      const float4 b = *reinterpret_cast<const float4 *>(p + 4);
      out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
      out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
  };
  if (single) {
    if (threadIdx.x < runs) {
      load_run(threadIdx.x, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  } else {
    for (int64_t r = threadIdx.x; r < runs; r += kThreads) {
      float t[8];
      load_run(r, t);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(t[i]));
    }
  }
  const float mx = block_max(amax, red);
  const float scale = mx / 127.0f;
  if (threadIdx.x == 0) sx[m] = scale;
  // The quotients x / scale from RN(1 / scale) and one correction step
  // (q8_code_rcp: the correctly rounded quotient wherever q8_row_rcp gives a
  // reciprocal, so the same codes), else the division itself.  The choice
  // is the same for the whole row.
  const float rc = q8_row_rcp(mx, scale);
  auto store_run = [&](int64_t r, const float *t) {
    uint32_t lo = 0, hi = 0;
    if (rc != 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= (static_cast<uint32_t>(static_cast<uint8_t>(q8_code_rcp(t[i], scale, rc))) << (8 * i));
        hi |= (static_cast<uint32_t>(static_cast<uint8_t>(q8_code_rcp(t[4 + i], scale, rc))) << (8 * i));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= (static_cast<uint32_t>(static_cast<uint8_t>(q8_code(t[i], scale))) << (8 * i));
        hi |= (static_cast<uint32_t>(static_cast<uint8_t>(q8_code(t[4 + i], scale))) << (8 * i));
      }
    }
    *reinterpret_cast<uint2 *>(xq + m * K + r * 8) = make_uint2(lo, hi);
  };
  if (single) {
    if (threadIdx.x < runs) store_run(threadIdx.x, v);
  } else {
    for (int64_t r = threadIdx.x; r < runs; r += kThreads) {
      float t[8];
      load_run(r, t);
      store_run(r, t);
    }
  }
}

// Element form for any K and alignment.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void quantize_rows_any(const void *__restrict__ x, int64_t K,
                                                              int8_t *__restrict__ xq,
                                                              float *__restrict__ sx) {
  __shared__ float red[kThreads / 64];
  const int64_t m = blockIdx.x;
  auto ld = [&](int64_t k) -> float {
    if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(x)[m * K + k]);
    else return static_cast<const float *>(x)[m * K + k];
  };
  float amax = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) amax = fmaxf(amax, fabsf(ld(k)));
  const float scale = block_max(amax, red) / 127.0f;
  if (threadIdx.x == 0) sx[m] = scale;
  for (int64_t k = threadIdx.x; k < K; k += kThreads) xq[m * K + k] = q8_code(ld(k), scale);
}

__global__ void zero_bytes(uint8_t *__restrict__ p, size_t n) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 16;
  if (i + 16 <= n && (reinterpret_cast<uintptr_t>(p + i) & 15) == 0) {
    *reinterpret_cast<uint4 *>(p + i) = make_uint4(0, 0, 0, 0);
  } else {
    for (size_t j = i; j < i + 16 && j < n; ++j) p[j] = 0;
  }
}

}  // namespace

hipError_t launch_zero(void *p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t per_block = 256 * 16;
  const unsigned blocks = static_cast<unsigned>((bytes + per_block - 1) / per_block);
  zero_bytes<<<blocks, 256, 0, st>>>(static_cast<uint8_t *>(p), bytes);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const void *x, bool x_bf16, int64_t M, int64_t K, int8_t *xq,
                                float *sx, hipStream_t st) {
  const bool vec = (K % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(xq) % 8 == 0);
  const dim3 grid(static_cast<unsigned>(M));
  if (vec) {
    if (x_bf16) quantize_rows_vec<true><<<grid, kThreads, 0, st>>>(x, K, xq, sx);
    else quantize_rows_vec<false><<<grid, kThreads, 0, st>>>(x, K, xq, sx);
  } else {
    if (x_bf16) quantize_rows_any<true><<<grid, kThreads, 0, st>>>(x, K, xq, sx);
    else quantize_rows_any<false><<<grid, kThreads, 0, st>>>(x, K, xq, sx);
  }
  return hipGetLastError();
}

}  // namespace q4
