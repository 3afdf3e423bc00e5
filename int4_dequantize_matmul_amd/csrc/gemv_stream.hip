// Decode GEMV for W4A16 (M <= 16): one streaming pass over the packed
// weights, in registers only.
//
// What it computes ("Fused int4 and int8 dequantize-matmul in C", sections
// 2.2-2.4, with bf16 activations and scales):
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]
// in f32, written as f32 and / or bf16 (round to nearest even).  A float
// path, judged by tolerance against the exact value.
//
// How (gfx950):
//   * A wave owns 4 weight rows.  Lane l covers k = 32 l .. 32 l + 31 of each
//     2048-wide pass, so one 16-byte load per lane reads 1 KB of a row,
//     contiguous: the wave streams its rows with no LDS and no barrier.
//   * A stored nibble u (two's complement storage turned into excess-8 by
//     u ^ 8) becomes the bf16 1 + u/16 exactly; v_dot2_f32_bf16 multiplies
//     pairs of those with the activation pairs.  Then
//       sum_k x (u - 8) = 16 * (sum_k x (1 + u/16) - sum_k 1.5 x)
//     per lane, times the lane's group scale (G a multiple of 32); the
//     second sum runs the same v_dot2 sequence against pairs of 1.5, so a
//     code 0 (u = 8) cancels exactly and a row of zero codes gives 0.  With
//     per-group zero points z ("The 4-bit CPU path", section W4A8: they
//     take the place of the constant 8) the stored u is used as is and
//       sum_k x (u - z) = 16 * (sum_k x (1 + u/16) - sum_k 1.5 x
//                               - ((z - 8)/24) sum_k 1.5 x).
//   * One workgroup serves every activation row (M <= 16), so the weights
//     are read once.  For M = 1 each lane loads its own activation slice,
//     and a workgroup is a single wave (measured faster than four: the
//     3328 waves of a 13312-row matrix spread more evenly over the CUs);
//     above that a workgroup of four waves stages the pass's activations in
//     LDS once for all of them.  Every
//     activation row goes through the same lane arithmetic and the same
//     fixed-order reduction over the 64 lanes, so a row's result does not
//     depend on M.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kRows = 4;              // weight rows per wave
constexpr int kWaves = 4;             // waves per workgroup (M >= 2: they share the staged activations)
constexpr int kWaves1 = 1;            // waves per workgroup at M = 1 (measured: smaller workgroups
                                      // balance the 3328 waves of a 13312-row matrix better)
constexpr int kLaneK = 32;            // k per lane per pass
constexpr int kPassK = 64 * kLaneK;   // k per pass: 2048

struct SArgs {
  const uint16_t *x;
  const uint8_t *w;
  const uint16_t *s;
  float *yf;          // may be null
  uint16_t *yb;       // may be null
  const uint8_t *z;   // zero points [N, K/G] (ZP kernels only)
  int M, N, K, Kb, G, Gn;
};

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Weights, group scales and zero points are read once per call: nontemporal
// loads keep them from displacing the activations in the caches (for the
// scales too this measured faster: 5.40 -> 5.13 us per call at N = 13312,
// K = 2048 over a cold pool).
__device__ __forceinline__ uint4 load16_stream(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p)));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

// Byte i of w (two excess-8 nibbles, low = even k) -> two bf16 1 + u/16:
// b * 0x8008 puts the low nibble at bits 3..6 and the high one at 19..22.
// The two masks arrive in registers so that the and-or is one instruction
// (a VOP3 operation takes no literal on this chip).
__device__ __forceinline__ uint32_t byte_to_bf16x2(uint32_t w, int i, uint32_t mask, uint32_t one) {
  uint32_t b = (w >> (8 * i)) & 0xFFu;
  if constexpr (Q4_MUTANT == 2) b = ((b & 0xFu) << 4) | (b >> 4);   // mutant s02: nibbles swapped
  return ((b * 0x8008u) & mask) | one;
}

__device__ __forceinline__ uint32_t dw4(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Sum over the 64 lanes in a fixed order; every lane ends with the total.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_row_sum_f32<16>(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// The arithmetic of one lane on one pass, shared by both kernels so that a
// row's bits do not depend on which of them ran it.
//
// The lane's activations against the bias weight: sum 1.5 x (pairs of bf16
// 1.5, the value 1 + 8/16 that a code 0 unpacks to), formed by the same
// v_dot2 sequence as a row's own sum, so that a run of codes 0 cancels to an
// exact zero (a row of zero codes gives y = 0, as its dequantized row does).
__device__ __forceinline__ float lane_xsum(const uint4 (&xv)[4]) {
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) v = dot2(dw4(xv[j >> 2], j & 3), 0x3FC03FC0u, v);   // pairs of bf16 1.5
  return v;
}

template <bool TW>
__device__ __forceinline__ void unpack_row(uint4 w, uint32_t (&wb)[16]) {
  constexpr uint32_t XM = TW ? 0x88888888u : 0u;   // two's complement storage -> excess-8
  uint32_t mask = 0x00780078u, one = 0x3F803F80u;
  asm("" : "+v"(mask), "+v"(one));   // opaque: keeps the constants in registers
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t wd = dw4(w, d) ^ XM;
#pragma unroll
    for (int i = 0; i < 4; ++i) wb[4 * d + i] = byte_to_bf16x2(wd, i, mask, one);   // k = 2j, 2j+1 for j = 4d+i
  }
}

// The lane's bias-corrected sum from its row sum d = sum x (1 + u/16) and
// the bias sum sx = sum 1.5 x of lane_xsum: d - sx = sum x (u - 8) / 16.
// With a zero point z the rest of its bias, (z - 8)/16 sum x = bz' sx with
// bz' = (z - 8)/24, comes off too: bz = -bz' (zp_bias), and z = 8 gives the
// symmetric result bit for bit.
template <bool ZP>
__device__ __forceinline__ float unbias(float d, float sx, float bz) {
  if constexpr (ZP) return fmaf(bz, sx, d - sx);
  else return Q4_MUTANT == 1 ? d - sx * (1.0f / 1.5f) : d - sx;   // mutant s01: u, not u - 8
}

// acc + 16 s (the lane's bias-corrected sum): acc + s sum x (u - 8) or
// acc + s sum x (u - z).
template <bool ZP>
__device__ __forceinline__ float lane_step(const uint4 (&xv)[4], const uint32_t (&wb)[16], float sx,
                                           float s16, float bz, float acc) {
  float d = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) d = dot2(dw4(xv[j >> 2], j & 3), wb[j], d);
  return fmaf(unbias<ZP>(d, sx, bz), s16, acc);
}

// -(z - 8)/24 for a 4-bit zero point z (rounded once; 0 for z = 8)
__device__ __forceinline__ float zp_bias(uint32_t z) { return (8.0f - static_cast<float>(z)) * (1.0f / 24.0f); }

template <int XB>
__device__ __forceinline__ void reduce_store(const SArgs &a, float (&acc)[XB][kRows], int lane, int n0) {
#pragma unroll
  for (int m = 0; m < XB; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[m][r] = wave_sum(acc[m][r]);
  if (lane != 0) return;
#pragma unroll
  for (int m = 0; m < XB; ++m) {
    if (m >= a.M) continue;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int n = n0 + r;
      if (n >= a.N) continue;
      const size_t o = static_cast<size_t>(m) * a.N + n;
      if (a.yf) a.yf[o] = acc[m][r];
      if (a.yb) a.yb[o] = f32_to_bf16_rne(acc[m][r]);
    }
  }
}

// M = 1: each lane loads its own activation slice.
template <bool TW, int XB, bool ZP>
__global__ __launch_bounds__(kWaves1 * 64) void gemv_stream_w4a16(SArgs a) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * kWaves1 + wv) * kRows;
  const int npass = (a.K + kPassK - 1) / kPassK;

  float acc[XB][kRows];
#pragma unroll
  for (int m = 0; m < XB; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[m][r] = 0.0f;

  // Registers of one pass: weights (16 B per row), group scales,
  // activations (64 B per row).  A scheduling barrier keeps every load of a
  // pass ahead of the arithmetic, so a wave has its whole pass in flight.
  // Loads complete in the order they were issued: the activations and each
  // row's scale go first, so the arithmetic of row r can start as soon as
  // row r's weights arrive.
  struct Pass {
    uint4 w[kRows];
    uint32_t sb[kRows];
    uint32_t zb[kRows];
    uint4 xv[XB][4];
  };
  auto fetch = [&](int p, Pass &f) {
    const int k0 = min(p * kPassK + lane * kLaneK, a.K - kLaneK);   // dead lanes re-read a live slice
#pragma unroll
    for (int m = 0; m < XB; ++m) {
      const uint16_t *xr = a.x + static_cast<size_t>(min(m, a.M - 1)) * a.K + k0;
#pragma unroll
      for (int i = 0; i < 4; ++i) f.xv[m][i] = load16(xr + 8 * i);
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int n = min(n0 + r, a.N - 1);
      f.sb[r] = __builtin_nontemporal_load(a.s + static_cast<size_t>(Q4_MUTANT == 3 ? 0 : n) * a.Gn + k0 / a.G);   // mutant s03: row 0's scales
      f.zb[r] = ZP ? __builtin_nontemporal_load(a.z + static_cast<size_t>(n) * a.Gn + k0 / a.G) : 8u;
      f.w[r] = load16_stream(a.w + static_cast<size_t>(n) * a.Kb + (Q4_MUTANT == 6 ? 0 : k0 / 2));   // mutant s06
    }
  };
  auto use = [&](int p, const Pass &c) {
    const bool live = p * kPassK + lane * kLaneK < a.K;   // K is a multiple of 32
    float sx[XB];
#pragma unroll
    for (int m = 0; m < XB; ++m) sx[m] = lane_xsum(c.xv[m]);
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      uint32_t wb[16];
      unpack_row<TW>(c.w[r], wb);
      const float s16 = 16.0f * bf16_to_f32(c.sb[r]);
      const float bz = ZP ? zp_bias(c.zb[r]) : 0.0f;   // (unused without zero points)
#pragma unroll
      for (int m = 0; m < XB; ++m) {
        float t = lane_step<ZP>(c.xv[m], wb, sx[m], s16, bz, acc[m][r]);
        if constexpr (Q4_MUTANT == 9) {   // mutant s09: M = 1 sums the lane's pairs in the opposite order
          float d = 0.0f;
#pragma unroll
          for (int j = 15; j >= 0; --j) d = dot2(dw4(c.xv[m][j >> 2], j & 3), wb[j], d);
          t = fmaf(unbias<ZP>(d, sx[m], bz), s16, acc[m][r]);
        }
        acc[m][r] = live ? t : acc[m][r];
      }
    }
  };

  // Two register sets used in turn: the next pass is in flight while the
  // current one is consumed, and no copy between the sets waits on a load.
  Pass A, B;
  fetch(0, A);
  int p = 0;
  for (; p + 2 < npass; p += 2) {
    fetch(p + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    use(p, A);
    fetch(p + 2, A);
    __builtin_amdgcn_sched_barrier(0);
    use(p + 1, B);
  }
  if (p + 1 < npass) {
    fetch(p + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    use(p, A);
    __builtin_amdgcn_sched_barrier(0);
    use(p + 1, B);
  } else {
    __builtin_amdgcn_sched_barrier(0);
    use(p, A);
  }
  reduce_store<XB>(a, acc, lane, n0);
}

// M = 2 .. 16: the workgroup copies the activation slice of a pass into LDS
// once ([row][chunk i][lane], so that each ds_read_b128 of a wave reads 1 KB
// of consecutive LDS), and every wave reads its lanes' slices from there.
template <bool TW, int XB, bool ZP>
__global__ __launch_bounds__(kWaves * 64) void gemv_stream_w4a16_lds(SArgs a) {
  __shared__ uint4 xs[XB][4][64];
  constexpr int kThreads = kWaves * 64;
  static_assert((XB * 256) % kThreads == 0, "the copy loop covers whole rows");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * kWaves + wv) * kRows;
  const int npass = (a.K + kPassK - 1) / kPassK;

  float acc[XB][kRows];
#pragma unroll
  for (int m = 0; m < XB; ++m)
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[m][r] = 0.0f;

  for (int p = 0; p < npass; ++p) {
    // activations first, so that waiting for them leaves the weights in flight
    uint4 xr[XB * 256 / kThreads];
#pragma unroll
    for (int i = 0; i < XB * 256 / kThreads; ++i) {
      const int c = threadIdx.x + i * kThreads;   // chunk c % 256 of row c / 256
      const int k = min(p * kPassK + 8 * (c & 255), a.K - 8);
      xr[i] = load16(a.x + static_cast<size_t>(min(c >> 8, a.M - 1)) * a.K + k);
    }
    const int k0 = min(p * kPassK + lane * kLaneK, a.K - kLaneK);
    uint4 w[kRows];
    uint32_t sb[kRows], zb[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int n = min(n0 + r, a.N - 1);
      w[r] = load16_stream(a.w + static_cast<size_t>(n) * a.Kb + (Q4_MUTANT == 6 ? 0 : k0 / 2));   // mutant s06
      sb[r] = __builtin_nontemporal_load(a.s + static_cast<size_t>(Q4_MUTANT == 3 ? 0 : n) * a.Gn + k0 / a.G);   // mutant s03
      zb[r] = ZP ? __builtin_nontemporal_load(a.z + static_cast<size_t>(n) * a.Gn + k0 / a.G) : 8u;
    }
    if (p > 0) lds_barrier();   // every wave is done with the previous slice
#pragma unroll
    for (int i = 0; i < XB * 256 / kThreads; ++i) {
      const int c = threadIdx.x + i * kThreads;
      xs[c >> 8][c & 3][(c & 255) >> 2] = xr[i];
    }
    lds_barrier();

    const bool live = p * kPassK + lane * kLaneK < a.K;
    uint32_t wb[kRows][16];
    float s16[kRows], bz[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      unpack_row<TW>(w[r], wb[r]);
      s16[r] = 16.0f * bf16_to_f32(sb[r]);
      bz[r] = ZP ? zp_bias(zb[r]) : 0.0f;   // (unused without zero points)
    }
#pragma unroll
    for (int m = 0; m < XB; ++m) {
      uint4 xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = xs[m][i][lane];
      const float sx = lane_xsum(xv);
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const float t = lane_step<ZP>(xv, wb[r], sx, s16[r], bz[r], acc[m][r]);
        acc[m][r] = live ? t : acc[m][r];
      }
    }
  }
  reduce_store<XB>(a, acc, lane, n0);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool TW, bool ZP>
hipError_t launch_stream(const SArgs &a, int64_t M, int64_t N, hipStream_t st) {
  if (M == 1) {
    const dim3 grid1(static_cast<unsigned>((N + kWaves1 * kRows - 1) / (kWaves1 * kRows)));
    gemv_stream_w4a16<TW, 1, ZP><<<grid1, kWaves1 * 64, 0, st>>>(a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((N + kWaves * kRows - 1) / (kWaves * kRows)));
  const int T = kWaves * 64;
  if (M == 2) gemv_stream_w4a16_lds<TW, 2, ZP><<<grid, T, 0, st>>>(a);
  else if (M <= 4) gemv_stream_w4a16_lds<TW, 4, ZP><<<grid, T, 0, st>>>(a);
  else if (M <= 8) gemv_stream_w4a16_lds<TW, 8, ZP><<<grid, T, 0, st>>>(a);
  else gemv_stream_w4a16_lds<TW, 16, ZP><<<grid, T, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

bool gemv_stream_w4a16_ok(const void *x, const void *wq, int64_t M, int64_t K, int64_t G) {
  return M >= 1 && M <= 16 && K > 0 && K % kLaneK == 0 && G > 0 && G % kLaneK == 0 && K % G == 0 &&
         aligned16(x) && aligned16(wq) && K < (int64_t(1) << 30);
}

hipError_t launch_gemv_stream_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                                    uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                                    hipStream_t st, const uint8_t *zp) {
  SArgs a{};
  a.x = x; a.w = wq; a.s = s; a.yf = yf; a.yb = yb; a.z = zp;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(K / 2);
  a.G = static_cast<int>(G);
  a.Gn = static_cast<int>(K / G);
  if (zp) return launch_stream<false, true>(a, M, N, st);   // zero points: the stored u as is
  if (enc == kTwos) return launch_stream<true, false>(a, M, N, st);
  return launch_stream<false, false>(a, M, N, st);
}

}  // namespace q4
