// Prefill: LDS-tiled bf16 MFMA GEMM for W4A16 (M >= 17).
//
// What it computes ("Fused int4 and int8 dequantize-matmul in C", sections
// 2.2 and 2.3, with bf16 activations and scales):
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]
// accumulated in f32 and written as f32 and / or bf16 (round to nearest
// even).  A float path: judged against the exact value by tolerance, so the
// group scale is applied with an FMA.
//
// How (gfx950):
//   * Workgroup tile 128 x 128 of y, 4 waves of 64 x 64; K in steps of 64
//     (a group of G = 64 j spans j steps).  Each step stages the activation
//     tile (128 x 64 bf16) and the unpacked weight tile (128 x 64 bf16) in
//     LDS, double-buffered: the next step's global loads are in flight while
//     the current step computes.  Two workgroups per CU.
//   * A stored nibble u (two's complement storage is first turned into
//     excess-8 by u ^ 8) becomes the bf16 1 + u/16, exactly, with one
//     multiply and one and-or per two values.  Then
//       sum_k x (u - 8) = 16 * (sum_k x (1 + u/16) - 1.5 sum_k x),
//     and the second sum, which depends on the row and the group only, is
//     formed by the threads that stage the activations (a v_dot2 chain over
//     the 32 values each holds, the two threads of a row added with a DPP
//     move), summed over the group's steps and handed to the fold through
//     LDS.  (Before, MFMAs against a constant -1.5 operand formed it: a
//     third of the kernel's MFMA work, 194 -> 177 us at the prefill shape.)  With
//     per-group zero points z ("The 4-bit CPU path", section W4A8: they
//     take the place of the constant 8) the group's fold scales the row sum
//     by 1 + z/16 of each column:
//       sum_k x (u - z) = 16 * (sum_k x (1 + u/16) - (1 + z/16) sum_k x).
//   * v_mfma_f32_32x32x16_bf16 for the products; LDS rows of 128 bytes with
//     the 16-byte chunk c of row r at position c ^ f(r), so that fragment
//     reads and staging writes touch distinct banks in every 8- and 16-lane
//     phase.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

// Cache policy of the output stores (sc0 | nt): y is written once and not
// read back, so it streams past the caches (measured: about 3% faster at
// the prefill shape).
constexpr int kStoreStream = 3;
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kTile = BM * BK * 2;            // one bf16 operand tile: 16 KB
constexpr int kOffB = kTile;                  // unpacked weights
constexpr int kOffS = 2 * kTile;              // 16 * group scale per column (f32)
constexpr int kOffX = kOffS + BN * 4;         // row sums of x over the group (f32), at its last step
constexpr int kOffZ = kOffX + BM * 4;         // zero points: 1 + z/16 per column (f32)
constexpr int stage_bytes(bool zp) { return kOffZ + (zp ? BN * 4 : 0); }

struct HArgs {
  const uint16_t *x;
  const uint8_t *w;
  const uint16_t *s;
  float *yf;          // may be null
  uint16_t *yb;       // may be null
  const uint8_t *z;   // zero points [N, K/G] (ZP kernels only)
  int M, N, K, Kb;
  int Gn, steps_per_group;
  int tiles_m, tiles_n;
  int remap;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz_f(int r) {
  return ((r & 3) ^ ((r >> 2) & 1)) | ((((r >> 2) ^ (r >> 3)) & 1) << 2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0), bytes,
                                           0x00020000);
}

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t dw4(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// D (32 x 32, f32) += A (32 x 16 bf16) * B (32 x 16 bf16)^T.  Operand lane l
// holds row (A) or column (B) l % 32, k = 8 (l / 32) .. +7 of the 16-wide k
// slice; result register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32.
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

// Byte i of w (two excess-8 nibbles, low = even k) -> two bf16 1 + u/16:
// b * 0x8008 puts the low nibble at bits 3..6 and the high one at 19..22.
__device__ __forceinline__ uint32_t byte_to_bf16x2(uint32_t w, int i) {
  const uint32_t b = (w >> (8 * i)) & 0xFFu;
  return ((b * 0x8008u) & 0x00780078u) | 0x3F803F80u;
}

template <bool TW, bool ZP>
__global__ __launch_bounds__(kThreads, 2) void tiled_w4a16_kernel(HArgs a) {
  constexpr uint32_t XM = TW ? 0x88888888u : 0u;   // two's complement storage -> excess-8
  constexpr int kStage = stage_bytes(ZP);
  __shared__ __align__(16) uint8_t st0[kStage], st1[kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;
  const int r32 = lane & 31, hi = lane >> 5;

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

  // ---- global -> registers (rows past M / N clamped) ----
  const __amdgpu_buffer_rsrc_t rs_x = rsrc(a.x, a.M * a.K * 2);
  const __amdgpu_buffer_rsrc_t rs_w = rsrc(a.w, a.N * a.Kb);
  const __amdgpu_buffer_rsrc_t rs_s = rsrc(a.s, a.N * a.Gn * 2);
  const int sr = tid >> 1, sh = tid & 1;       // tile row, half of the step (32 k)
  const int fr = swz_f(sr);
  const int x_voff = min(m0 + sr, a.M - 1) * (a.K * 2) + sh * 64;
  const int w_voff = min(n0 + sr, a.N - 1) * a.Kb + sh * 16;
  const int s_voff = min(n0 + (tid & (BN - 1)), a.N - 1) * a.Gn * 2;
  const __amdgpu_buffer_rsrc_t rs_z = rsrc(a.z, ZP ? a.N * a.Gn : 0);
  const int z_voff = min(n0 + (tid & (BN - 1)), a.N - 1) * a.Gn;
  uint4 ra[4], rb;
  uint32_t rsv = 0, rzv = 8;
  float xg = 0.0f;   // this row's sum of x over the current group (both halves of the row)
  auto gload = [&](int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = bload16(rs_x, x_voff + i * 16, s * BK * 2);
    rb = bload16(rs_w, w_voff, s * (BK / 2));
    rsv = __builtin_amdgcn_raw_buffer_load_b16(rs_s, s_voff, (s / a.steps_per_group) * 2, 0);
    if constexpr (ZP) rzv = __builtin_amdgcn_raw_buffer_load_b8(rs_z, z_voff, s / a.steps_per_group, 0);
  };
  // s: the step whose data ra / rb hold
  auto lstore = [&](uint8_t *st, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4 *>(st + sr * 128 + (((sh * 4 + i) ^ fr) << 4)) = ra[i];
    // the row's sum of x over this step (32 values per thread, then the two
    // threads of the row, adjacent lanes), added to the group's sum; at the
    // group's last step it goes to LDS for the fold
    float xs = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) xs = dot2_bf16(dw4(ra[j >> 2], j & 3), 0x3F803F80u, xs);
    xs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, xs), 0xB1, 0xF, 0xF, false));
    xg += xs;
    if ((s + 1) % a.steps_per_group == 0) {
      if (sh == 0) reinterpret_cast<float *>(st + kOffX)[sr] = xg;
      xg = 0.0f;
    }
    // 16 packed bytes (32 nibbles, k order) -> 64 bytes of bf16 1 + u/16
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = dw4(rb, c) ^ XM;
      *reinterpret_cast<uint4 *>(st + kOffB + sr * 128 + (((sh * 4 + c) ^ fr) << 4)) =
          make_uint4(byte_to_bf16x2(w, 0), byte_to_bf16x2(w, 1), byte_to_bf16x2(w, 2), byte_to_bf16x2(w, 3));
    }
    if (tid < BN) {
      const int col = tid;
      const int pos = ((col >> 6) * 32 + (col & 31)) * 2 + ((col >> 5) & 1);
      reinterpret_cast<float *>(st + kOffS)[pos] = 16.0f * bf16_to_f32(rsv & 0xFFFFu);
      if constexpr (ZP) reinterpret_cast<float *>(st + kOffZ)[pos] = 1.0f + static_cast<float>(rzv & 0xFFu) * 0.0625f;
    }
  };

  // ---- fragments: lane l reads row (column) l % 32 of its block, chunk
  // 2 * slice + l / 32; slice j sits at the slice-0 address ^ 32 j ----
  const int fl = swz_f(r32);
  const int a_base = (wm * 64 + r32) * 128 + ((hi ^ fl) << 4);
  const int b_base = kOffB + (wn * 64 + r32) * 128 + ((hi ^ fl) << 4);
  const int s_off = kOffS + (wn * 32 + r32) * 8;
  // this lane's output rows 8 j + 4 hi + 0..3 of block mb: their x sums
  const int x_off = kOffX + (wm * 64 + 4 * hi) * 4;

  f32x16 acc[2][2];
  float t[2][2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      acc[mb][nb] = f32x16{};
#pragma unroll
      for (int r = 0; r < 16; ++r) t[mb][nb][r] = 0.0f;
    }
  }

  auto mma = [&](const uint8_t *cur) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 Af[2][2], Bf[2][2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int x = 32 * (2 * h + jj);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) Af[jj][mb] = *reinterpret_cast<const uint4 *>(cur + (a_base ^ x) + mb * 4096);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) Bf[jj][nb] = *reinterpret_cast<const uint4 *>(cur + (b_base ^ x) + nb * 4096);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma_bf16_32x32x16(Af[jj][mb], Bf[jj][nb], acc[mb][nb]);
    }
  };
  // end of a group: t += 16 s (D - 1.5 sum x), or with zero points
  // t += 16 s (D - (1 + z/16) sum x); then clear the group sums
  auto fold = [&](const uint8_t *cur) {
    const float2 sv = *reinterpret_cast<const float2 *>(cur + s_off);
    const float sc[2] = {sv.x, sv.y};
    float zf[2] = {1.0f, 1.0f};
    if constexpr (ZP) {
      const float2 zv = *reinterpret_cast<const float2 *>(cur + s_off + (kOffZ - kOffS));
      zf[0] = zv.x;
      zf[1] = zv.y;
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float xr[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 v = *reinterpret_cast<const float4 *>(cur + x_off + (mb * 32 + 8 * j) * 4);
        xr[4 * j] = v.x; xr[4 * j + 1] = v.y; xr[4 * j + 2] = v.z; xr[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float cb = ZP ? -zf[nb] : -1.5f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float d = fmaf(cb, xr[r], acc[mb][nb][r]);
          t[mb][nb][r] = fmaf(d, sc[nb], t[mb][nb][r]);
        }
        acc[mb][nb] = f32x16{};
      }
    }
  };

  gload(0);
  lstore(st0, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const uint8_t *cur = (s & 1) ? st1 : st0;
    uint8_t *nxt = (s & 1) ? st0 : st1;
    gload(min(s + 1, nsteps - 1));
    mma(cur);
    if ((s + 1) % a.steps_per_group == 0) fold(cur);
    lstore(nxt, s + 1);   // past the last step: reloads step nsteps - 1, unused
    __syncthreads();
  }

  // ---- output: f32 and / or bf16 (RNE).  Buffer stores whose bounds end
  // at y[M-1][N-1] (from this wave's first element): rows past M fall
  // outside, columns past N get an offset far outside, and the hardware
  // drops those stores. ----
  const int mrow0 = m0 + wm * 64, ncol0 = n0 + wn * 64;
  const int64_t rem = static_cast<int64_t>(a.M - mrow0) * a.N - ncol0;
  const int64_t nel = rem > 0 ? min(rem, static_cast<int64_t>(64) * a.N) : 0;
  const size_t base = rem > 0 ? static_cast<size_t>(mrow0) * a.N + ncol0 : 0;
  const __amdgpu_buffer_rsrc_t rs_yf = rsrc(a.yf ? a.yf + base : nullptr, a.yf ? static_cast<int>(nel * 4) : 0);
  const __amdgpu_buffer_rsrc_t rs_yb = rsrc(a.yb ? a.yb + base : nullptr, a.yb ? static_cast<int>(nel * 2) : 0);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int col = nb * 32 + r32;
    const bool col_ok = ncol0 + col < a.N;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * mb + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int e = col_ok ? row * a.N + col : (1 << 28);   // element offset; far outside when past N
        const float v = t[mb][nb][r];
        if (a.yf) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs_yf, e * 4, 0, kStoreStream);
        if (a.yb) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), rs_yb, e * 2, 0, kStoreStream);
      }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool tiled_w4a16_ok(const void *x, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G) {
  if (M < 17 || K <= 0 || K % BK != 0 || G <= 0 || G % BK != 0 || K % G != 0) return false;
  if (!aligned16(x) || !aligned16(wq)) return false;
  if (M * K * 2 >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31)) return false;
  if (N * (K / G) * 2 >= (int64_t(1) << 31)) return false;
  if (256 * N >= (int64_t(1) << 29)) return false;   // byte offsets within 64 rows stay below 2^29
  return true;
}

int64_t tiled_w4a16_tiles(int64_t M, int64_t N) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

hipError_t launch_tiled_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf, uint16_t *yb,
                              int64_t M, int64_t N, int64_t K, int64_t G, int enc, hipStream_t st,
                              const uint8_t *zp) {
  HArgs a{};
  a.x = x; a.w = wq; a.s = s; a.yf = yf; a.yb = yb; a.z = zp;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(K / 2);
  a.Gn = static_cast<int>(K / G);
  a.steps_per_group = static_cast<int>(G / BK);
  a.tiles_m = static_cast<int>((M + BM - 1) / BM);
  a.tiles_n = static_cast<int>((N + BN - 1) / BN);
  a.remap = (a.tiles_n % 8 == 0) ? 1 : 0;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.tiles_m) * a.tiles_n));
  if (zp) tiled_w4a16_kernel<false, true><<<grid, kThreads, 0, st>>>(a);   // zero points: the stored u as is
  else if (enc == kTwos) tiled_w4a16_kernel<true, false><<<grid, kThreads, 0, st>>>(a);
  else tiled_w4a16_kernel<false, false><<<grid, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace q4
