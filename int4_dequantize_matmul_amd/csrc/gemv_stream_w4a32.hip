// GEMV for W4A32: f32 activations against packed int4 weights with one f16
// scale per group of G columns.
//
// What it computes ("Fused int4 and int8 dequantize-matmul in C", sections
// 2.2-2.4 and the worked example of section 3):
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]
// accumulated in f32: a float path, judged by tolerance against the exact
// value.
//
// How (gfx950):
//   * A wave owns R weight rows.  Lane l covers columns 32 l .. 32 l + 31 of
//     each 2048-wide pass, so one 16-byte nontemporal load per row and lane
//     reads 1 KB of a row per wave instruction, contiguous.  The lane's 32
//     columns lie in one group (G is a multiple of 32), so each lane needs
//     one scale per row and pass.
//   * Nibbles become floats with no per-nibble shift: t = stored ^ XM puts
//     the code in excess-8 form u = q + 8 (two's complement: XM = 0x88..88),
//     t & 0x0F0F0F0F holds the even columns' u and (t >> 4) & 0x0F0F0F0F
//     the odd columns', one per byte, and v_cvt_f32_ubyte turns each byte
//     into f32(u) exactly.  Then
//       sum_{lane's k} x q = sum x u - 8 sum x,
//     and acc += s * (that): one FMA per weight, about 2.25 VALU
//     instructions per weight in all.
//   * A workgroup is one wave and serves XB activation rows (1 or 2); more
//     rows take more workgroups along y, each with the same lane arithmetic
//     and the same fixed-order reduction over the 64 lanes, so a row's bits
//     do not depend on M.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kLaneK = 32;            // columns per lane per pass
constexpr int kPassK = 64 * kLaneK;   // columns per pass: 2048
constexpr int kMaxXB = 2;             // activation rows per workgroup

struct A32Args {
  const float *x;       // [M, K]
  const uint8_t *w;     // [N, K/2]
  const uint16_t *s;    // [N, K/G] f16 bits
  float *y;             // [M, N]
  int M, N, K, G;
};

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16_stream(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p)));
}

__device__ __forceinline__ uint32_t dw4(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Column c (0..31) of the lane's activations, held as 8 dwordx4.
__device__ __forceinline__ float xcol(const uint4 (&xv)[8], int c) {
  return __uint_as_float(dw4(xv[c >> 2], c & 3));
}

// f32 of byte i of w; the compiler selects one v_cvt_f32_ubyte<i>.
__device__ __forceinline__ float ubyte_f32(uint32_t w, int i) {
  return static_cast<float>((w >> (8 * i)) & 0xFFu);
}

__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_row_sum_f32<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// One lane, one pass, one weight row, one activation row: sum x u over the
// lane's 32 columns (u = q + 8).
template <bool TW>
__device__ __forceinline__ float lane_dot(const uint4 (&xv)[8], uint4 wv) {
  constexpr uint32_t XM = TW ? 0x88888888u : 0u;
  float d = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {              // dword j: columns 8 j .. 8 j + 7
    const uint32_t t = dw4(wv, j) ^ XM;
    const uint32_t lo = t & 0x0F0F0F0Fu;         // columns 8 j + 0, 2, 4, 6
    const uint32_t hi = (t >> 4) & 0x0F0F0F0Fu;  // columns 8 j + 1, 3, 5, 7
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      d = fmaf(xcol(xv, 8 * j + 2 * b), ubyte_f32(lo, b), d);
      d = fmaf(xcol(xv, 8 * j + 2 * b + 1), ubyte_f32(hi, b), d);
    }
  }
  return d;
}

template <bool TW, int XB, int R>
__global__ __launch_bounds__(64) void gemv_stream_w4a32(A32Args a) {
  const int lane = threadIdx.x;
  const int n0 = blockIdx.x * R;
  const int m0 = blockIdx.y * XB;
  const int npass = (a.K + kPassK - 1) / kPassK;
  const int Kb = a.K / 2;
  const int Gn = a.K / a.G;

  float acc[XB][R];
#pragma unroll
  for (int m = 0; m < XB; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  for (int p = 0; p < npass; ++p) {
    const int kl = p * kPassK + lane * kLaneK;
    const bool live = kl < a.K;               // K is a multiple of 32
    const int k0 = min(kl, a.K - kLaneK);      // dead lanes re-read a live slice
    // activations, then scales, then weights: loads complete in issue
    // order, so the arithmetic of row r starts when its weights arrive
    uint4 xv[XB][8];
#pragma unroll
    for (int m = 0; m < XB; ++m) {
      const float *xr = a.x + static_cast<size_t>(min(m0 + m, a.M - 1)) * a.K + k0;
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[m][i] = load16(xr + 4 * i);
    }
    uint32_t sb[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      // nontemporal, as the weights: read once per call (3.32 -> 3.20 us per call)
      sb[r] = __builtin_nontemporal_load(a.s + static_cast<size_t>(min(n0 + r, a.N - 1)) * Gn + k0 / a.G);
    uint4 w[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      w[r] = load16_stream(a.w + static_cast<size_t>(min(n0 + r, a.N - 1)) * Kb + k0 / 2);
    __builtin_amdgcn_sched_barrier(0);
    float sx[XB];
#pragma unroll
    for (int m = 0; m < XB; ++m) {
      float v = 0.0f;
#pragma unroll
      for (int c = 0; c < kLaneK; ++c) v += xcol(xv[m], c);
      sx[m] = v;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float s = Q4_MUTANT == 5 ? bf16_to_f32(sb[r]) : f16_to_f32(sb[r]);   // mutant s05: f16 read as bf16
#pragma unroll
      for (int m = 0; m < XB; ++m) {
        const float d = fmaf(-8.0f, sx[m], lane_dot<TW>(xv[m], w[r]));
        acc[m][r] = live ? fmaf(s, d, acc[m][r]) : acc[m][r];
      }
    }
  }

#pragma unroll
  for (int m = 0; m < XB; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = wave_sum(acc[m][r]);
  if (lane != 0) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = n0 + r;
    if (n >= a.N) continue;
#pragma unroll
    for (int m = 0; m < XB; ++m)
      if (m0 + m < a.M) a.y[static_cast<size_t>(m0 + m) * a.N + n] = acc[m][r];
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool TW, int R>
hipError_t launch_r(const A32Args &a, int64_t M, int64_t N, hipStream_t st) {
  const unsigned gx = static_cast<unsigned>((N + R - 1) / R);
  if (M == 1) gemv_stream_w4a32<TW, 1, R><<<dim3(gx, 1), 64, 0, st>>>(a);
  else gemv_stream_w4a32<TW, kMaxXB, R><<<dim3(gx, static_cast<unsigned>((M + kMaxXB - 1) / kMaxXB)), 64, 0, st>>>(a);
  return hipGetLastError();
}

// Rows per wave: enough waves to fill the chip at the small matrices this
// format is used for (2048 rows give 1024 workgroups).
template <bool TW>
hipError_t launch_tw(const A32Args &a, int64_t M, int64_t N, hipStream_t st) {
  if (N >= 8192) return launch_r<TW, 4>(a, M, N, st);
  if (N >= 1024) return launch_r<TW, 2>(a, M, N, st);
  return launch_r<TW, 1>(a, M, N, st);
}

}  // namespace

bool gemv_stream_w4a32_ok(const void *x, const void *wq, int64_t M, int64_t K, int64_t G) {
  return M >= 1 && (M + kMaxXB - 1) / kMaxXB <= 65535 && K > 0 && G > 0 && G % kLaneK == 0 && K % G == 0 &&
         aligned16(x) && aligned16(wq) && K < (int64_t(1) << 28);
}

hipError_t launch_gemv_stream_w4a32(const float *x, const uint8_t *wq, const uint16_t *s, float *y, int64_t M,
                                    int64_t N, int64_t K, int64_t G, int enc, hipStream_t st) {
  A32Args a{};
  a.x = x; a.w = wq; a.s = s; a.y = y;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K); a.G = static_cast<int>(G);
  return enc == kTwos ? launch_tw<true>(a, M, N, st) : launch_tw<false>(a, M, N, st);
}

}  // namespace q4
