// General kernels: every shape the API accepts, any alignment.
//
// They read the packed bytes one at a time and decode each nibble with the
// plain rules (two's complement: u < 8 ? u : u - 16; excess-8: u - 8;
// "Fused int4 and int8 dequantize-matmul in C", section 2.2, and
// ftts_kernels module int4, "Packing").  One wave owns one weight row n and
// a block of up to 16 activation rows, so every output has a single owner
// and a fixed summation order (section 2.5 of the same page: one worker per
// output, threads never change the bits).
//
// Float activations: y[m,n] = sum_k x[m,k] * (q[n,k] * s[n,k/G]).  The
// product q*s is exact in f32 (4-bit code times an 11-bit or 8-bit scale
// significand), so this is the factored sum of section 2.3 up to the
// rounding of the f32 accumulation.
//
// With per-group zero points z[n, k/G] ("The 4-bit CPU path", section W4A8:
// a checkpoint's zero points take the place of the constant 8) the code is
// q = u - z for the stored nibble u, in [-15, 15]; q*s stays exact in f32.
//
// Integer activations: exact i32 sums, then the fixed f32 epilogue:
//   per channel  y = (f32(acc) * sx[m]) * sw[n]
//   grouped      t = f32(acc_0) s_0; t = t + f32(acc_g) s_g, g increasing;
//                y = t * sx[m]
// (ftts_kernels module int8, module head: scales once, after accumulation,
// in a fixed order).  Compiled with -ffp-contract=off: no FMA in it.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kWaves = 4;
constexpr int kMB = 16;  // activation rows per wave

__device__ __forceinline__ int decode_nibble(uint32_t u, int enc) {
  return enc == kExcess8 ? static_cast<int>(u) - 8 : (u < 8 ? static_cast<int>(u) : static_cast<int>(u) - 16);
}

// Code of nibble u at column k of row n: with zero points u - z[n, k/G].
__device__ __forceinline__ int weight_code(uint32_t u, int enc, const uint8_t *zp, int64_t n, int64_t Gn,
                                           int64_t k, int64_t G) {
  return zp ? static_cast<int>(u) - static_cast<int>(zp[n * Gn + k / G]) : decode_nibble(u, enc);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <bool XBF16, bool SBF16>
__global__ __launch_bounds__(kWaves * 64) void generic_float(
    const void *__restrict__ x, const uint8_t *__restrict__ wq, const uint16_t *__restrict__ s,
    float *__restrict__ yf, uint16_t *__restrict__ yb, int64_t M, int64_t N, int64_t K,
    int64_t G, int enc, const uint8_t *__restrict__ zp) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (n >= N) return;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kMB;
  const int Mb = static_cast<int>(M - m0 < kMB ? M - m0 : kMB);
  const int64_t Kb = K / 2, Gn = K / G;
  const uint8_t *row = wq + n * Kb;
  float acc[kMB];
#pragma unroll
  for (int m = 0; m < kMB; ++m) acc[m] = 0.0f;
  for (int64_t b = lane; b < Kb; b += 64) {
    const uint32_t byte = row[b];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t k = 2 * b + h;
      const uint32_t u = h ? (byte >> 4) : (byte & 0xFu);
      const uint32_t sb = s[n * Gn + k / G];
      const float sc = SBF16 ? bf16_to_f32(sb) : f16_to_f32(sb);
      const float w = static_cast<float>(weight_code(u, enc, zp, n, Gn, k, G)) * sc;  // exact
#pragma unroll
      for (int m = 0; m < kMB; ++m) {
        if (m < Mb) {
          float xv;
          if constexpr (XBF16) xv = bf16_to_f32(static_cast<const uint16_t *>(x)[(m0 + m) * K + k]);
          else xv = static_cast<const float *>(x)[(m0 + m) * K + k];
          acc[m] = fmaf(xv, w, acc[m]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kMB; ++m) {
    if (m < Mb) {
      const float v = wave_sum_f32(acc[m]);
      if (lane == 0) {
        if (yf) yf[(m0 + m) * N + n] = v;
        if (yb) yb[(m0 + m) * N + n] = f32_to_bf16_rne(v);
      }
    }
  }
}

template <bool W8>
__global__ __launch_bounds__(kWaves * 64) void generic_int(
    const int8_t *__restrict__ xq, const float *__restrict__ sx, const void *__restrict__ w,
    const float *__restrict__ sw, float *__restrict__ y, int64_t M, int64_t N, int64_t K,
    int64_t G, int enc, const uint8_t *__restrict__ zp) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (n >= N) return;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kMB;
  const int Mb = static_cast<int>(M - m0 < kMB ? M - m0 : kMB);
  const int64_t rb = W8 ? K : (K + 1) / 2;
  const uint8_t *row = static_cast<const uint8_t *>(w) + n * rb;
  const int64_t Gz = G > 0 ? K / G : 1;
  auto weight = [&](int64_t k) -> int {
    if constexpr (W8) return static_cast<int8_t>(row[k]);
    const uint32_t byte = row[k >> 1];
    return weight_code((k & 1) ? (byte >> 4) : (byte & 0xFu), enc, zp, n, Gz, k, G > 0 ? G : K);
  };
  if (G == 0) {
    int acc[kMB];
#pragma unroll
    for (int m = 0; m < kMB; ++m) acc[m] = 0;
    for (int64_t k = lane; k < K; k += 64) {
      const int wk = weight(k);
#pragma unroll
      for (int m = 0; m < kMB; ++m)
        if (m < Mb) acc[m] += static_cast<int>(xq[(m0 + m) * K + k]) * wk;
    }
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
      if (m < Mb) {
        const int a = wave_sum_i32(acc[m]);
        if (lane == 0) {
          const float t = static_cast<float>(a) * sx[m0 + m];
          y[(m0 + m) * N + n] = t * sw[n];
        }
      }
    }
    return;
  }
  const int64_t Gn = K / G;
  float t[kMB];
#pragma unroll
  for (int m = 0; m < kMB; ++m) t[m] = 0.0f;
  for (int64_t g = 0; g < Gn; ++g) {
    int acc[kMB];
#pragma unroll
    for (int m = 0; m < kMB; ++m) acc[m] = 0;
    for (int64_t k = g * G + lane; k < (g + 1) * G; k += 64) {
      const int wk = weight(k);
#pragma unroll
      for (int m = 0; m < kMB; ++m)
        if (m < Mb) acc[m] += static_cast<int>(xq[(m0 + m) * K + k]) * wk;
    }
    const float sg = sw[n * Gn + g];
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
      if (m < Mb) {
        const int a = wave_sum_i32(acc[m]);   // every lane holds the exact total
        const float p = static_cast<float>(a) * sg;
        t[m] = (g == 0) ? p : t[m] + p;
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < kMB; ++m)
      if (m < Mb) y[(m0 + m) * N + n] = t[m] * sx[m0 + m];
  }
}

// int8 weights with one f32 scale per row against float activations:
// y[m,n] = s[n] * sum_k x[m,k] q[n,k], f32 accumulation.
template <bool XBF16>
__global__ __launch_bounds__(kWaves * 64) void generic_w8_float(
    const void *__restrict__ x, const int8_t *__restrict__ wq, const float *__restrict__ s,
    float *__restrict__ yf, uint16_t *__restrict__ yb, int64_t M, int64_t N, int64_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (n >= N) return;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kMB;
  const int Mb = static_cast<int>(M - m0 < kMB ? M - m0 : kMB);
  const int8_t *row = wq + n * K;
  float acc[kMB];
#pragma unroll
  for (int m = 0; m < kMB; ++m) acc[m] = 0.0f;
  for (int64_t k = lane; k < K; k += 64) {
    const float q = static_cast<float>(row[k]);
#pragma unroll
    for (int m = 0; m < kMB; ++m) {
      if (m < Mb) {
        float xv;
        if constexpr (XBF16) xv = bf16_to_f32(static_cast<const uint16_t *>(x)[(m0 + m) * K + k]);
        else xv = static_cast<const float *>(x)[(m0 + m) * K + k];
        acc[m] = fmaf(xv, q, acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < kMB; ++m) {
    if (m < Mb) {
      const float v = wave_sum_f32(acc[m]) * s[n];
      if (lane == 0) {
        if (yf) yf[(m0 + m) * N + n] = v;
        if (yb) yb[(m0 + m) * N + n] = f32_to_bf16_rne(v);
      }
    }
  }
}

dim3 generic_grid(int64_t M, int64_t N) {
  return dim3(static_cast<unsigned>((N + kWaves - 1) / kWaves),
              static_cast<unsigned>((M + kMB - 1) / kMB));
}

}  // namespace

hipError_t launch_generic_float(const void *x, bool x_bf16, const uint8_t *wq, const uint16_t *s,
                                bool s_bf16, float *yf, uint16_t *yb, int64_t M, int64_t N,
                                int64_t K, int64_t G, int enc, hipStream_t st, const uint8_t *zp) {
  const dim3 grid = generic_grid(M, N);
  if (x_bf16 && s_bf16)
    generic_float<true, true><<<grid, kWaves * 64, 0, st>>>(x, wq, s, yf, yb, M, N, K, G, enc, zp);
  else if (!x_bf16 && !s_bf16)
    generic_float<false, false><<<grid, kWaves * 64, 0, st>>>(x, wq, s, yf, yb, M, N, K, G, enc, zp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_generic_int(const int8_t *xq, const float *sx, const void *w, bool w_int8,
                              const float *sw, float *y, int64_t M, int64_t N, int64_t K,
                              int64_t G, int enc, hipStream_t st, const uint8_t *zp) {
  const dim3 grid = generic_grid(M, N);
  if (w_int8)
    generic_int<true><<<grid, kWaves * 64, 0, st>>>(xq, sx, w, sw, y, M, N, K, 0, enc, nullptr);
  else
    generic_int<false><<<grid, kWaves * 64, 0, st>>>(xq, sx, w, sw, y, M, N, K, G, enc, zp);
  return hipGetLastError();
}

hipError_t launch_generic_w8_float(const void *x, bool x_bf16, const int8_t *wq, const float *s, float *yf,
                                   uint16_t *yb, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const dim3 grid = generic_grid(M, N);
  if (x_bf16) generic_w8_float<true><<<grid, kWaves * 64, 0, st>>>(x, wq, s, yf, yb, M, N, K);
  else generic_w8_float<false><<<grid, kWaves * 64, 0, st>>>(x, wq, s, yf, yb, M, N, K);
  return hipGetLastError();
}

}  // namespace q4
