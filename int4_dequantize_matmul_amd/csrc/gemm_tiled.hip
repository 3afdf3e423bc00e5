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
//   * Workgroup tile 128 x 128 of y, 4 waves of 64 x 64 on
//     v_mfma_i32_32x32x32_i8 (the full-rate int8 shape); K in steps of 128
//     (one weight group per step in the grouped form).  Each step stages
//     the activation tile (128 x 128 int8) and the weight tile (128 rows x
//     64 packed bytes) through registers into LDS, double-buffered.  Per
//     channel two register sets keep the loads of the next two steps in
//     flight while a step computes; grouped, the running sums need those
//     registers and the loads run one step ahead.  The barriers wait for
//     LDS traffic only, so they never drain outstanding loads.
//   * The packed weights are unpacked once per workgroup into LDS as signed
//     bytes holding 16*q: each nibble is moved to the top half of its byte
//     (the two's-complement code q then reads as the int8 16*q).  That costs
//     a shift, two masks and two byte permutes per 8 nibbles, and leaves no
//     +8 bias to cancel: the MFMA sums are exactly 16*acc.
//       per channel  f32(16*acc) * 2^-4 = f32(acc) exactly, then the two
//                    scale multiplies;
//       grouped      f32(16*acc_g) * (s_g * 2^-4) is the product acc_g*s_g
//                    rounded once, provided s_g * 2^-4 is exact.  A scale so
//                    small that it is not (|s| < 2^-122) flags its step, and
//                    that step takes f32(16*acc_g >> 4) * s_g instead.
//   * Per-group zero points z ("The 4-bit CPU path", section W4A8: they take
//     the place of the constant 8; grouped only): the weights are unpacked
//     to the signed bytes u - z instead, as ((u + (0x80 - z)) ^ 0x80) per
//     byte (u + 0x80 - z lies in 113..143, so no carry crosses a byte).  The
//     MFMA sums are then acc_g itself and the epilogue multiplies by s_g.
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at
//     position c ^ f(r), with f chosen so that every 8- and 16-lane phase of
//     a fragment read and of a staging write touches distinct banks.
//   * The grouped epilogue is 3 VALU ops per output per group (convert,
//     multiply, add); the running sum starts at -0.0, the identity of f32
//     addition, so the first group needs no special case.  Two workgroups
//     per CU let one wave's epilogue run beside another wave's MFMAs.
//   * Tiles are ordered so that each XCD (workgroup id mod 8) owns a band of
//     weight columns and walks all activation rows: its weights stay in its
//     L2 while the activation tiles stream through.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kTile = BM * BK;                  // one operand tile, int8 (16 KB)
// One pipeline stage: A tile | unpacked B tile | [grouped: scales/16 | scales | 2 flags]
constexpr int kOffB = kTile;
constexpr int kOffS16 = 2 * kTile;
constexpr int kOffS = kOffS16 + BN * 4;
constexpr int kOffFlag = kOffS + BN * 4;
constexpr int kStageG = kOffFlag + 16;
constexpr int kStageC = 2 * kTile;
constexpr int lds_bytes(bool grouped) { return 2 * (grouped ? kStageG : kStageC) + (BM + BN) * 4; }

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
  const uint8_t *z;  // per-group zero points [N, K/G] (ZP kernel only)
};

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Chunk position permutation of row r (depends on r mod 16 only).
__device__ __forceinline__ int swz_f(int r) {
  return ((r & 3) ^ ((r >> 2) & 1)) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int bytes) {
  // raw buffer, bounds = bytes; dword 3 as for gfx9 raw buffers
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

typedef int i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ i32x16 mfma_i8_32x32x32(uint4 a, uint4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t dw4(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <bool GROUPED, bool TW, bool ZP>
__global__ __launch_bounds__(kThreads, 2) void tiled_w4a8_kernel(TArgs a) {
  static_assert(!ZP || (GROUPED && !TW), "zero points: grouped, stored nibbles used as is");
  constexpr int kStage = GROUPED ? kStageG : kStageC;
  // excess-8 storage becomes two's complement under u ^ 8
  constexpr uint32_t XM = TW ? 0u : 0x88888888u;
  constexpr uint32_t MF0 = 0xF0F0F0F0u;
  extern __shared__ __align__(16) uint8_t smem[];
  float *Sx = reinterpret_cast<float *>(smem + 2 * kStage);   // [BM]
  float *Sw = Sx + BM;                                          // [BN] per-channel scales

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;

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

  if (tid < BM) Sx[tid] = a.sx[min(m0 + tid, a.M - 1)];
  else if (!GROUPED) Sw[tid - BM] = a.sw[min(n0 + tid - BM, a.N - 1)];

  // ---- global -> register staging (rows past M / N clamped) ----
  const __amdgpu_buffer_rsrc_t rs_a = rsrc(a.xq, a.M * a.K);
  const __amdgpu_buffer_rsrc_t rs_b = rsrc(a.w, a.N * a.Kb);
  const __amdgpu_buffer_rsrc_t rs_s = rsrc(a.sw, GROUPED ? a.N * a.Gn * 4 : 4);
  const int sr = tid >> 1, sh = tid & 1;     // row of the tile, half of the step
  const int fr = swz_f(sr);
  const int a_voff = min(m0 + sr, a.M - 1) * a.K + sh * 64;
  const int b_voff = min(n0 + sr, a.N - 1) * a.Kb + sh * 32;
  const int s_voff = GROUPED ? min(n0 + (tid & (BN - 1)), a.N - 1) * a.Gn * 4 : 0;
  const __amdgpu_buffer_rsrc_t rs_z = rsrc(a.z, ZP ? a.N * a.Gn : 0);
  const int z_voff = ZP ? min(n0 + sr, a.N - 1) * a.Gn : 0;   // zero point of this thread's weight row
  // One step's operands in registers on their way to LDS.
  struct Stg {
    uint4 ra[4], rb[2];
    float rsv;
    uint32_t rz;
  };
  auto gload = [&](int s, Stg &g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) g.ra[i] = bload16(rs_a, a_voff + i * 16, s * BK);
#pragma unroll
    for (int i = 0; i < 2; ++i) g.rb[i] = bload16(rs_b, b_voff + i * 16, s * (BK / 2));
    if constexpr (GROUPED)
      g.rsv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_s, s_voff, s * 4, 0));
    else
      g.rsv = 0.0f;
    if constexpr (ZP) g.rz = __builtin_amdgcn_raw_buffer_load_b8(rs_z, z_voff, s, 0);   // group s (G == BK)
    else g.rz = 0u;
  };
  auto lstore = [&](uint8_t *st, const Stg &g) {
    const uint4 *ra = g.ra, *rb = g.rb;
    const float rsv = g.rsv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4 *>(st + sr * 128 + (((sh * 4 + i) ^ fr) << 4)) = ra[i];
    // 32 packed bytes -> 64 bytes of 16*q (or u - z) in k order: chunk c
    // from dwords 2c, 2c+1
    const uint32_t cz = ZP ? (0x80u - (g.rz & 0xFFu)) * 0x01010101u : 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w = dw4(rb[c >> 1], (c & 1) * 2 + h);
        uint32_t lo, hi;
        if constexpr (ZP) {
          lo = ((w & 0x0F0F0F0Fu) + cz) ^ 0x80808080u;
          hi = (((w >> 4) & 0x0F0F0F0Fu) + cz) ^ 0x80808080u;
        } else {
          lo = ((w << 4) ^ (XM << 4)) & MF0;
          hi = (w ^ XM) & MF0;
        }
        o[2 * h] = perm_b32(hi, lo, 0x05010400u);       // k+0..3
        o[2 * h + 1] = perm_b32(hi, lo, 0x07030602u);   // k+4..7
      }
      *reinterpret_cast<uint4 *>(st + kOffB + sr * 128 + (((sh * 4 + c) ^ fr) << 4)) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
    if constexpr (GROUPED) {
      if (tid < BN) {   // waves 0 and 1: one column each
        const int col = tid;
        const int pos = ((col >> 6) * 32 + (col & 31)) * 2 + ((col >> 5) & 1);
        // the fast slot holds the factor of the MFMA sum: s / 16 for 16 acc,
        // s itself for the zero-point form (whose sums are acc)
        const float s16 = ZP ? rsv : rsv * 0.0625f;
        const bool inexact = ZP ? false : !(s16 * 16.0f == rsv);
        reinterpret_cast<float *>(st + kOffS16)[pos] = s16;
        reinterpret_cast<float *>(st + kOffS)[pos] = rsv;
        const uint64_t bad = __ballot(inexact);
        if (lane == 0) reinterpret_cast<uint32_t *>(st + kOffFlag)[wv] = bad != 0 ? 1u : 0u;
      }
    }
  };

  // ---- fragment addresses (stage-relative) ----
  // v_mfma_i32_32x32x32_i8: lane l supplies row (A) or column (B) l % 32 and
  // the 16 k bytes 16 (l / 32) .. of the 32-wide k slice; k slice kk of the
  // step is chunk 2 kk + l / 32 of the row.
  // Chunk 2 kk + h of row r sits at position (2 kk + h) ^ f(r); the row
  // base is 128-byte aligned, so slice kk's address is slice 0's ^ 32 kk.
  const int l32 = lane & 31, lh = lane >> 5;
  const int fl = swz_f(l32);
  const int a_off0 = (wm * 64 + l32) * 128 + ((lh ^ fl) << 4);
  const int b_off0 = kOffB + (wn * 64 + l32) * 128 + ((lh ^ fl) << 4);
  const int s_off = (wn * 32 + l32) * 8;

  // acc[mb][nb] is the 32 x 32 block (mb, nb) of the wave's 64 x 64 tile:
  // register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
  i32x16 acc[2][2];
  float t[2][2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[mb][nb][r] = 0;
        t[mb][nb][r] = -0.0f;
      }
    }

  auto mma = [&](const uint8_t *cur) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 Af[2], Bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        Af[i] = *reinterpret_cast<const uint4 *>(cur + ((a_off0 ^ (kk << 5)) + i * 32 * 128));
        Bf[i] = *reinterpret_cast<const uint4 *>(cur + ((b_off0 ^ (kk << 5)) + i * 32 * 128));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const i32x16 zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
          const i32x16 c0 = (GROUPED && kk == 0) ? zero : acc[mb][nb];
          acc[mb][nb] = mfma_i8_32x32x32(Af[mb], Bf[nb], c0);
        }
    }
  };
  // t = t + f32(acc_g) * s_g
  auto epi_fast = [&](const uint8_t *cur) {
    const float2 sv = *reinterpret_cast<const float2 *>(cur + kOffS16 + s_off);
    const float sc[2] = {sv.x, sv.y};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = static_cast<float>(acc[mb][nb][r]) * sc[nb];
          t[mb][nb][r] = t[mb][nb][r] + p;
        }
  };
  auto epi_exact = [&](const uint8_t *cur) {
    const float2 sv = *reinterpret_cast<const float2 *>(cur + kOffS + s_off);
    const float sc[2] = {sv.x, sv.y};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = static_cast<float>(acc[mb][nb][r] >> 4) * sc[nb];
          t[mb][nb][r] = t[mb][nb][r] + p;
        }
  };
  // One K step on stage `cur`; the other stage receives the next step's
  // data.  Per channel that data was requested one step earlier and the
  // step after it is requested now (two register sets); grouped, it is
  // requested at the start of the step.  The last steps reload the last
  // step's data into the idle stage (never read again), which keeps every
  // step free of branches around loads and stores.  The barrier waits for
  // LDS traffic only, so requests for later steps stay in flight.
  auto compute = [&](const uint8_t *cur) {
    if constexpr (GROUPED) {
      const uint2 fv = *reinterpret_cast<const uint2 *>(cur + kOffFlag);
      if (__builtin_amdgcn_readfirstlane(fv.x | fv.y) == 0) {
        mma(cur);
        epi_fast(cur);
      } else {
        mma(cur);
        epi_exact(cur);
      }
    } else {
      mma(cur);
    }
  };

  Stg g0, g1;
  if constexpr (GROUPED) {
    // the running sums take the registers a second staging set would need
    gload(0, g0);
    lstore(smem, g0);
    lds_barrier();
    for (int s = 0; s < nsteps; ++s) {
      const int o = (s & 1) * kStage;
      gload(min(s + 1, nsteps - 1), g0);
      compute(smem + o);
      lstore(smem + (kStage - o), g0);
      lds_barrier();
    }
  } else {
    gload(0, g0);
    gload(min(1, nsteps - 1), g1);
    lstore(smem, g0);
    lds_barrier();
    for (int s = 0; s < nsteps; s += 2) {
      // even step: stage 0 computes, g1 (step s + 1) goes to stage 1
      gload(min(s + 2, nsteps - 1), g0);
      compute(smem);
      lstore(smem + kStage, g1);
      lds_barrier();
      if (s + 1 >= nsteps) break;
      // odd step: stage 1 computes, g0 (step s + 2) goes to stage 0
      gload(min(s + 3, nsteps - 1), g1);
      compute(smem + kStage);
      lstore(smem, g0);
      lds_barrier();
    }
  }

  // ---- epilogue: y = t * sx (grouped) or ((f32(16 acc) / 16) * sx) * sw ----
  // Stores go through a buffer whose bounds end at y[M-1][N-1] (counted from
  // this wave's first element, at most 64 rows): rows past M fall outside it,
  // columns past N get an offset far outside it, and the hardware drops
  // those stores.
  const int mrow0 = m0 + wm * 64, ncol0 = n0 + wn * 64;
  const int64_t rem = static_cast<int64_t>(a.M - mrow0) * a.N - ncol0;
  const int nrec = rem > 0 ? static_cast<int>(min(rem, static_cast<int64_t>(64) * a.N) * 4) : 0;
  const __amdgpu_buffer_rsrc_t rs_y =
      rsrc(a.y + (rem > 0 ? static_cast<size_t>(mrow0) * a.N + ncol0 : 0), nrec);
  int vcol[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int c = nb * 32 + l32;
    vcol[nb] = (ncol0 + c < a.N) ? c * 4 : (1 << 30);
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);   // wave-relative row
      const float sxr = Sx[wm * 64 + rl];
      const int roff = rl * a.N * 4;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float v;
        if constexpr (GROUPED) {
          v = t[mb][nb][r] * sxr;
        } else {
          const float f = static_cast<float>(acc[mb][nb][r]) * 0.0625f;
          v = (f * sxr) * Sw[wn * 64 + nb * 32 + l32];
        }
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs_y, roff + vcol[nb], 0, 0);
      }
    }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool tiled_w4a8_ok(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G) {
  if (M < 17 || K <= 0 || K % BK != 0 || !(G == 0 || G == BK)) return false;
  if (!aligned16(xq) || !aligned16(wq)) return false;
  // 32-bit buffer offsets; 16*acc must fit i32 over all of K per channel
  if (M * K >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31)) return false;
  if (G && N * (K / G) * 4 >= (int64_t(1) << 31)) return false;
  if (!G && K > 131072) return false;
  if (256 * N >= (int64_t(1) << 30)) return false;   // y offsets within 64 rows stay below 2^30
  return true;
}

hipError_t launch_tiled_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                             float *y, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                             hipStream_t st, const uint8_t *zp) {
  TArgs a{};
  a.xq = xq; a.sx = sx; a.w = wq; a.sw = sw; a.y = y;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(K / 2);
  a.Gn = G ? static_cast<int>(K / G) : 0;
  a.tiles_m = static_cast<int>((M + BM - 1) / BM);
  a.tiles_n = static_cast<int>((N + BN - 1) / BN);
  const int64_t tiles = static_cast<int64_t>(a.tiles_m) * a.tiles_n;
  a.remap = (a.tiles_n % 8 == 0) ? 1 : 0;
  const dim3 grid(static_cast<unsigned>(tiles));
  static const bool attrs = [] {
    // more than 64 KB of dynamic LDS per workgroup must be allowed explicitly
    bool ok = true;
    for (const void *k : {reinterpret_cast<const void *>(tiled_w4a8_kernel<true, true, false>),
                          reinterpret_cast<const void *>(tiled_w4a8_kernel<true, false, false>),
                          reinterpret_cast<const void *>(tiled_w4a8_kernel<true, false, true>)})
      ok &= hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes(true)) == hipSuccess;
    for (const void *k : {reinterpret_cast<const void *>(tiled_w4a8_kernel<false, true, false>),
                          reinterpret_cast<const void *>(tiled_w4a8_kernel<false, false, false>)})
      ok &= hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes(false)) == hipSuccess;
    return ok;
  }();
  if (!attrs) return hipErrorInvalidValue;
  if (zp) {
    a.z = zp;
    tiled_w4a8_kernel<true, false, true><<<grid, kThreads, lds_bytes(true), st>>>(a);
  } else if (G) {
    if (enc == kTwos) tiled_w4a8_kernel<true, true, false><<<grid, kThreads, lds_bytes(true), st>>>(a);
    else tiled_w4a8_kernel<true, false, false><<<grid, kThreads, lds_bytes(true), st>>>(a);
  } else {
    if (enc == kTwos) tiled_w4a8_kernel<false, true, false><<<grid, kThreads, lds_bytes(false), st>>>(a);
    else tiled_w4a8_kernel<false, false, false><<<grid, kThreads, lds_bytes(false), st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace q4
