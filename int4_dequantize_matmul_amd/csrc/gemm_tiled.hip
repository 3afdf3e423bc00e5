// Prefill: LDS-tiled int8 MFMA GEMM for W4A8 (M >= 17).
//
// What it computes (ftts_kernels module int4, "Packing" / linear_q4, and
// module int8 head; "Fused int4 and int8 dequantize-matmul in C", section
// 2.3 for the grouped form):
//   per channel  acc = sum_k xq[m,k] q[n,k] (exact i32);  y = (f32(acc)*sx)*sw
//   grouped      acc_g exact per group of 128;  t = f32(acc_0)*s_0, then
//                t = t + f32(acc_g)*s_g in increasing g;  y = t*sx
// bit for bit, with no FMA in the epilogue.
//
// How (gfx950):
//   * Workgroup tile 128 x 128 of y, 4 waves of 64 x 64; K in steps of 128.
//     Each step stages the activation tile (128 x 128 int8) and the weight
//     tile (128 rows x 64 packed bytes) into LDS, double-buffered: the next
//     step's global loads are in flight while the current step computes.
//   * The packed weights are unpacked once per workgroup into LDS as the
//     stored nibble values u (bytes 0..15) in natural k order:
//       lo = w & 0x0F0F0F0F, hi = (w >> 4) & 0x0F0F0F0F, two byte perms.
//     The stored +8 bias cancels on the matrix core: an MFMA of the
//     activation fragment with a constant -8 operand gives -8 * sum xq over
//     the group, which seeds the accumulator of the main MFMAs, so that
//     acc = sum xq (u - 8) = sum xq q exactly.
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at
//     position c ^ ((r >> 1) & 7), so a 16-lane phase of a fragment read
//     touches all banks once.
//   * The grouped epilogue is 3 VALU ops per output per group (convert,
//     multiply, add); the running sum starts at -0.0, the identity of f32
//     addition, so the first group needs no special case.  The epilogue is
//     the bound of this kernel: it is more VALU work than the int8 MFMAs are
//     matrix-core work, and two workgroups per CU let one wave's epilogue run
//     beside another wave's MFMAs.
//   * Tiles are ordered so that each XCD (workgroup id mod 8) owns a band of
//     weight columns and walks all activation rows: its weights stay in its
//     L2 while the activation tiles stream through.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kStageBytes = BM * BK;              // one operand tile, int8
constexpr int kLdsFixed = 4 * kStageBytes + 2 * BM * 4;   // A,B double-buffered + sx + sw

struct TArgs {
  const int8_t *xq;
  const float *sx;
  const uint8_t *w;
  const float *sw;
  float *y;
  int M, N, K, Kb;
  int Gn;          // groups per row (grouped), 0 per channel
  int tiles_m, tiles_n;
  int remap;       // reorder tiles by XCD
};

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ uint32_t dw4(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <bool GROUPED, bool TW>
__global__ __launch_bounds__(kThreads, 2) void tiled_w4a8_kernel(TArgs a) {
  constexpr uint32_t XM = TW ? 0x88888888u : 0u;
  constexpr uint32_t M0F = 0x0F0F0F0Fu;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t *As = smem;                                   // [2][128 rows m][128 B]
  uint8_t *Bs = smem + 2 * kStageBytes;                 // [2][128 rows n][128 B]
  float *Sx = reinterpret_cast<float *>(smem + 4 * kStageBytes);   // [128]
  float *Sw = Sx + BM;                                  // [128] per-channel scales
  float *Sg = Sw + BN;                                  // [128][Gn] group scales

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;
  const int l16 = lane & 15, lg = lane >> 4;

  // XCD e (= workgroup id mod 8) owns weight-column tiles [e*pn, (e+1)*pn)
  // and walks them fastest, so the tiles it runs at one time share
  // activation rows and its weights stay in its L2.
  int m_tile, n_tile;
  if (a.remap) {
    const int pn = a.tiles_n >> 3, l = blockIdx.x >> 3;
    n_tile = (blockIdx.x & 7) * pn + l % pn;
    m_tile = l / pn;
  } else {
    m_tile = blockIdx.x % a.tiles_m;
    n_tile = blockIdx.x / a.tiles_m;
  }
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int nsteps = a.K / BK;

  // ---- scales of this tile into LDS ----
  if (tid < BM) Sx[tid] = a.sx[min(m0 + tid, a.M - 1)];
  if constexpr (!GROUPED) {
    if (tid < BN) Sw[tid] = a.sw[min(n0 + tid, a.N - 1)];
  } else {
    const size_t base = static_cast<size_t>(n0) * a.Gn, last = static_cast<size_t>(a.N) * a.Gn - 1;
    for (int e = tid; e < BN * a.Gn; e += kThreads) Sg[e] = a.sw[min(base + e, last)];
  }

  // ---- global -> register staging assignment (rows past M / N clamped) ----
  const int sr = tid >> 1, sh = tid & 1;     // row of the tile, half of the step
  const int8_t *a_src = a.xq + static_cast<size_t>(min(m0 + sr, a.M - 1)) * a.K + sh * 64;
  const uint8_t *b_src = a.w + static_cast<size_t>(min(n0 + sr, a.N - 1)) * a.Kb + sh * 32;
  uint4 ra[4], rb[2];
  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = load16(a_src + s * BK + i * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) rb[i] = load16(b_src + s * (BK / 2) + i * 16);
  };
  auto lstore = [&](int stage) {
    uint8_t *as = As + stage * kStageBytes;
    uint8_t *bs = Bs + stage * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(as + swz(sr, sh * 4 + i)) = ra[i];
    // 32 packed bytes -> 64 nibble bytes in k order
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t o[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t w = dw4(rb[i], d) ^ XM;
        const uint32_t lo = w & M0F, hi = (w >> 4) & M0F;
        o[2 * d] = perm_b32(hi, lo, 0x05010400u);       // k+0..3
        o[2 * d + 1] = perm_b32(hi, lo, 0x07030602u);   // k+4..7
      }
      *reinterpret_cast<uint4 *>(bs + swz(sr, sh * 4 + 2 * i)) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4 *>(bs + swz(sr, sh * 4 + 2 * i + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  const uint4 CB = make_uint4(0xF8F8F8F8u, 0xF8F8F8F8u, 0xF8F8F8F8u, 0xF8F8F8F8u);   // int8 -8
  i32x4 acc[4][4];
  i32x4 bias[4];
  float t[4][4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    bias[mb] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      acc[mb][nb] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) t[mb][nb][r] = -0.0f;
    }
  }

  gload(0);
  lstore(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int stage = s & 1;
    if (s + 1 < nsteps) gload(s + 1);
    const uint8_t *as = As + stage * kStageBytes;
    const uint8_t *bs = Bs + stage * kStageBytes;
    // activation fragments of both k halves
    uint4 Af[2][4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        Af[kh][mb] = *reinterpret_cast<const uint4 *>(as + swz(wm * 64 + mb * 16 + l16, kh * 4 + lg));
    // -8 * sum of the activations over this step, per row
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      i32x4 b0 = GROUPED ? i32x4{0, 0, 0, 0} : bias[mb];
      b0 = mfma_i8_16x16x64(Af[0][mb], CB, b0);
      bias[mb] = mfma_i8_16x16x64(Af[1][mb], CB, b0);
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      uint4 Bf[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        Bf[nb] = *reinterpret_cast<const uint4 *>(bs + swz(wn * 64 + nb * 16 + l16, kh * 4 + lg));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const i32x4 c = (GROUPED && kh == 0) ? bias[mb] : acc[mb][nb];
          acc[mb][nb] = mfma_i8_16x16x64(Af[kh][mb], Bf[nb], c);
        }
    }
    if constexpr (GROUPED) {
      // t = t + f32(acc_g) * s_g   (group g = step s)
      float sc[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) sc[nb] = Sg[(wn * 64 + nb * 16 + l16) * a.Gn + s];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = static_cast<float>(acc[mb][nb][r]) * sc[nb];
            t[mb][nb][r] = t[mb][nb][r] + p;
          }
    }
    if (s + 1 < nsteps) lstore(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: y = t * sx (grouped) or (f32(acc) * sx) * sw ----
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int rb0 = wm * 64 + mb * 16 + lg * 4;          // first of this lane's 4 rows
    const float4 sxv = *reinterpret_cast<const float4 *>(Sx + rb0);
    const float sxr[4] = {sxv.x, sxv.y, sxv.z, sxv.w};
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = wn * 64 + nb * 16 + l16;
      const int n = n0 + col;
      float swc = 0.f;
      if constexpr (!GROUPED) swc = Sw[col];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + rb0 + r;
        float yv;
        if constexpr (GROUPED) {
          yv = t[mb][nb][r] * sxr[r];
        } else {
          const float tt = static_cast<float>(acc[mb][nb][r] + bias[mb][r]) * sxr[r];
          yv = tt * swc;
        }
        if (m < a.M && n < a.N) a.y[static_cast<size_t>(m) * a.N + n] = yv;
      }
    }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool tiled_w4a8_ok(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G) {
  if (M < 17 || K <= 0 || K % BK != 0 || !(G == 0 || G == BK)) return false;
  if (!aligned16(xq) || !aligned16(wq)) return false;
  const int64_t gn = G ? K / G : 0;
  const size_t lds = kLdsFixed + static_cast<size_t>(BN * gn) * 4;
  return lds <= 80 * 1024 && M < (int64_t(1) << 31) && N < (int64_t(1) << 31);
}

hipError_t launch_tiled_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                             float *y, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                             hipStream_t st) {
  TArgs a{};
  a.xq = xq; a.sx = sx; a.w = wq; a.sw = sw; a.y = y;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(K / 2);
  a.Gn = G ? static_cast<int>(K / G) : 0;
  a.tiles_m = static_cast<int>((M + BM - 1) / BM);
  a.tiles_n = static_cast<int>((N + BN - 1) / BN);
  const int64_t tiles = static_cast<int64_t>(a.tiles_m) * a.tiles_n;
  a.remap = (a.tiles_n % 8 == 0) ? 1 : 0;
  const size_t lds = kLdsFixed + static_cast<size_t>(BN * a.Gn) * 4;
  const dim3 grid(static_cast<unsigned>(tiles));
  static const bool attrs = [] {
    // more than 64 KB of dynamic LDS per workgroup must be allowed explicitly
    const int lim = 96 * 1024;
    bool ok = hipFuncSetAttribute(reinterpret_cast<const void *>(tiled_w4a8_kernel<true, true>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, lim) == hipSuccess;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void *>(tiled_w4a8_kernel<true, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lim) == hipSuccess;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void *>(tiled_w4a8_kernel<false, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lim) == hipSuccess;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void *>(tiled_w4a8_kernel<false, false>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lim) == hipSuccess;
    return ok;
  }();
  if (!attrs) return hipErrorInvalidValue;
  if (G) {
    if (enc == kTwos) tiled_w4a8_kernel<true, true><<<grid, kThreads, lds, st>>>(a);
    else tiled_w4a8_kernel<true, false><<<grid, kThreads, lds, st>>>(a);
  } else {
    if (enc == kTwos) tiled_w4a8_kernel<false, true><<<grid, kThreads, lds, st>>>(a);
    else tiled_w4a8_kernel<false, false><<<grid, kThreads, lds, st>>>(a);
  }
  return hipGetLastError();
}

bool tiled_w4a16_ok(const void *, const void *, int64_t, int64_t, int64_t, int64_t) { return false; }
hipError_t launch_tiled_w4a16(const uint16_t *, const uint8_t *, const uint16_t *, float *, uint16_t *,
                              int64_t, int64_t, int64_t, int64_t, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace q4
