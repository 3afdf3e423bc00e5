// GEMV with int8 weights and float activations (W8A32, W8A16).
//
// What it computes ("Fused int4 and int8 dequantize-matmul in C", section 4,
// tl_matmul_q8_f32, and the int8 form of the worked example in section 3;
// ftts_kernels module int8, linear_w8a16):
//   y[m,n] = s[n] * sum_k x[m,k] q[n,k]
// with int8 codes q, one f32 scale per weight row, f32 x (W8A32) or bf16 x
// (W8A16), accumulated in f32.  A float path, judged by tolerance.
//
// How (gfx950):
//   * A wave owns 4 weight rows.  Lane l covers k = 16 l .. 16 l + 15 of each
//     1024-wide pass, so one 16-byte nontemporal load per row and lane reads
//     1 KB of a row per wave instruction, contiguous.
//   * A code q becomes the unsigned byte u = q ^ 0x80 = q + 128, and
//     v_cvt_f32_ubyte turns it into f32(u) exactly; then
//       sum_k x q = sum_k x u - 128 sum_k x.
//     bf16 x: u has at most 8 significant bits, so the top half of f32(u) is
//     u in bf16, and two of them form one v_dot2_f32_bf16 operand.  f32 x:
//     one v_fmac_f32 per weight.
//   * A workgroup serves up to 4 activation rows (more rows take more
//     workgroups along y); every row goes through the same lane arithmetic
//     and the same fixed-order reduction over the 64 lanes, so a row's bits
//     do not depend on M.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kRows = 4;              // weight rows per wave
constexpr int kWaves = 4;             // waves per workgroup
constexpr int kLaneK = 16;            // k per lane per pass
constexpr int kPassK = 64 * kLaneK;   // k per pass: 1024
constexpr int kMaxXB = 4;             // activation rows per workgroup

struct W8Args {
  const void *x;      // [M, K] f32 or bf16 bits
  const int8_t *w;    // [N, K]
  const float *s;     // [N]
  float *yf;          // may be null (W8A16)
  uint16_t *yb;       // W8A16 only
  int M, N, K;
};

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load16_stream(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p)));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

__device__ __forceinline__ uint32_t dw4(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_row_sum_f32<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// f32(u) of byte i of w (u = the stored int8 code + 128); the compiler
// selects one v_cvt_f32_ubyte<i> for this pattern.
__device__ __forceinline__ float ubyte_f32(uint32_t w, int i) {
  return static_cast<float>((w >> (8 * i)) & 0xFFu);
}

// One lane, one pass, one weight row, one activation row: sum x u - 128 sum x.
template <bool XBF16>
__device__ __forceinline__ float lane_dot(const uint4 (&xv)[4], uint4 wv, float sx) {
  float d = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t u = dw4(wv, j) ^ 0x80808080u;            // k = 4 j .. 4 j + 3
    const float f0 = ubyte_f32(u, 0), f1 = ubyte_f32(u, 1), f2 = ubyte_f32(u, 2), f3 = ubyte_f32(u, 3);
    if constexpr (XBF16) {
      // bf16 pairs (f0, f1), (f2, f3): the top halves of the exact f32 values
      const uint32_t b01 = perm_b32(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      const uint32_t b23 = perm_b32(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
      d = dot2(dw4(xv[j >> 1], (j & 1) * 2), b01, d);
      d = dot2(dw4(xv[j >> 1], (j & 1) * 2 + 1), b23, d);
    } else {
      const uint4 xj = xv[j];
      d = fmaf(__uint_as_float(xj.x), f0, d);
      d = fmaf(__uint_as_float(xj.y), f1, d);
      d = fmaf(__uint_as_float(xj.z), f2, d);
      d = fmaf(__uint_as_float(xj.w), f3, d);
    }
  }
  return fmaf(-128.0f, sx, d);
}

// sum of this lane's 16 activations
template <bool XBF16>
__device__ __forceinline__ float lane_xsum(const uint4 (&xv)[4]) {
  float v = 0.0f;
  if constexpr (XBF16) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v = dot2(dw4(xv[j >> 2], j & 3), 0x3F803F80u, v);   // pairs of bf16 1.0
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v += __uint_as_float(dw4(xv[j >> 2], j & 3));
  }
  return v;
}

template <bool XBF16, int XB>
__global__ __launch_bounds__(kWaves * 64) void gemv_stream_w8(W8Args a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * kWaves + wv) * kRows;
  const int m0 = blockIdx.y * XB;
  const int npass = (a.K + kPassK - 1) / kPassK;
  constexpr int XBYTES = XBF16 ? 2 : 4;

  float acc[XB][kRows];
#pragma unroll
  for (int m = 0; m < XB; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[m][r] = 0.0f;

  for (int p = 0; p < npass; ++p) {
    const int kl = p * kPassK + lane * kLaneK;
    const bool live = kl < a.K;                 // K is a multiple of 16
    const int k0 = min(kl, a.K - kLaneK);        // dead lanes re-read a live slice
    // activations first: loads complete in issue order, so row r's
    // arithmetic can start as soon as its weights arrive
    uint4 xv[XB][4];
#pragma unroll
    for (int m = 0; m < XB; ++m) {
      const uint8_t *xr = static_cast<const uint8_t *>(a.x) +
                          (static_cast<size_t>(min(m0 + m, a.M - 1)) * a.K + k0) * XBYTES;
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[m][i] = (XBF16 && i >= 2) ? make_uint4(0u, 0u, 0u, 0u) : load16(xr + 16 * i);
    }
    uint4 w[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int n = min(n0 + r, a.N - 1);
      w[r] = load16_stream(a.w + static_cast<size_t>(n) * a.K + k0);
    }
    __builtin_amdgcn_sched_barrier(0);
    float sx[XB];
#pragma unroll
    for (int m = 0; m < XB; ++m) sx[m] = lane_xsum<XBF16>(xv[m]);
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int m = 0; m < XB; ++m) {
        const float d = lane_dot<XBF16>(xv[m], w[r], sx[m]);
        acc[m][r] = live ? acc[m][r] + d : acc[m][r];
      }
  }

#pragma unroll
  for (int m = 0; m < XB; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[m][r] = wave_sum(acc[m][r]);
  if (lane != 0) return;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int n = n0 + r;
    if (n >= a.N) continue;
    const float sc = a.s[n];
#pragma unroll
    for (int m = 0; m < XB; ++m) {
      if (m0 + m >= a.M) continue;
      const size_t o = static_cast<size_t>(m0 + m) * a.N + n;
      const float y = acc[m][r] * sc;
      if (a.yf) a.yf[o] = y;
      if (a.yb) a.yb[o] = f32_to_bf16_rne(y);
    }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool XBF16>
hipError_t launch_w8(const W8Args &a, int64_t M, int64_t N, hipStream_t st) {
  const unsigned gx = static_cast<unsigned>((N + kWaves * kRows - 1) / (kWaves * kRows));
  const int T = kWaves * 64;
  if (M == 1) gemv_stream_w8<XBF16, 1><<<dim3(gx, 1), T, 0, st>>>(a);
  else if (M == 2) gemv_stream_w8<XBF16, 2><<<dim3(gx, 1), T, 0, st>>>(a);
  else gemv_stream_w8<XBF16, kMaxXB><<<dim3(gx, static_cast<unsigned>((M + kMaxXB - 1) / kMaxXB)), T, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

bool gemv_stream_w8_ok(const void *x, const void *wq, int64_t M, int64_t K) {
  return M >= 1 && (M + kMaxXB - 1) / kMaxXB <= 65535 && K > 0 && K % kLaneK == 0 && aligned16(x) &&
         aligned16(wq) && K < (int64_t(1) << 28);
}

hipError_t launch_gemv_stream_w8(const void *x, bool x_bf16, const int8_t *wq, const float *s, float *yf,
                                 uint16_t *yb, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  W8Args a{};
  a.x = x; a.w = wq; a.s = s; a.yf = yf; a.yb = yb;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  return x_bf16 ? launch_w8<true>(a, M, N, st) : launch_w8<false>(a, M, N, st);
}

}  // namespace q4
