// Prefill: LDS-tiled bf16 MFMA GEMM for W4A16 (M >= 17), staged by loads
// that write LDS.
//
// What it computes ("Fused int4 and int8 dequantize-matmul in C", sections
// 2.2 and 2.3, with bf16 activations and scales):
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]
// accumulated in f32 and written as f32 and / or bf16 (round to nearest
// even).  A float path, judged against the exact value by tolerance.
//
// How (gfx950):
//   * Workgroup tile 128 x 128, four waves of 64 x 64 (2 x 2), K in steps of
//     64 (a group of G = 64 j spans j steps), two workgroups per CU.  The
//     tiles past the last whole round of workgroups run as two 64-row
//     halves, waves of 32 x 64, in the same launch: the last round then
//     fills the slots with short pieces.  A small call (at most 64 rows,
//     or four 64 x 64 pieces per tile fit one round of workgroups) runs as
//     64 x 64 pieces, waves of 32 x 32.
//   * Staging: the activation tile (128 rows x 128 bytes of bf16), the
//     packed weight tile (128 rows x 32 bytes) and the step's group scales
//     go from global memory straight into LDS with buffer loads that write
//     LDS, into a ring of three stages, issued two steps ahead; one barrier
//     per step.  No registers hold staged data.
//   * Operands of v_mfma_f32_32x32x16_bf16: in k slice j (0..3) of a step,
//     lane (r, h) takes k = 32 h + 8 j .. + 7, for the activation row r of
//     its block (16 bytes of LDS) and for the weight column r (4 packed
//     bytes: one 16-byte LDS read per column gives all four slices).  The
//     MFMA sums whatever k its two lane halves hold, so the four slices cover
//     the step's 64 k once.
//   * Unpack in registers by each wave for its own 64 columns: a stored
//     nibble u (two's complement storage turned into excess-8 by u ^ 8)
//     becomes the bf16 1 + u/16 exactly, then
//       sum_k x (u - 8) = 16 (sum_k x (1 + u/16) - 1.5 sum_k x);
//     the activation sums of the wave's rows come from the same fragments
//     (v_dot2 against 1.0), over the group, and reach the output layout
//     through a small LDS area of the wave's own.  With zero points z the
//     1.5 becomes 1 + z/16 of each column.
//   * At a group's end t = fma(fma(-1.5, sum x, D), 16 s, t); the next
//     group's first products start from zero (an inline-constant operand).
//   * LDS: chunk c of activation row r sits at c ^ f(r), so every 8-lane
//     phase of a fragment read touches distinct banks.
#include <type_traits>

#include "kernels.hpp"
#include "q4_device.hpp"
#include "q4_lds_dma.hpp"

namespace q4 {
namespace {

// Cache policy of the output stores (sc0 | nt): y is written once and not
// read back, so it streams past the caches.
constexpr int kStoreStream = 3;
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int NS = 3;                      // LDS ring stages
constexpr int kA = BM * BK * 2;            // activation tile: 16 KB
constexpr int kB = BN * BK / 2;            // packed weight tile: 4 KB
constexpr int kS = 4 * 64 * 4;             // scales: 4 waves x 64 lanes x 4-byte slots
constexpr int kZ = 4 * 64 * 4;             // zero points (ZP): one byte per lane's slot
constexpr int stage_bytes(bool zp) { return kA + kB + kS + (zp ? kZ : 0); }
constexpr int kRS = 4 * 2 * 32 * 4;        // each wave's row sums: 2 blocks x 32 rows
constexpr int lds_bytes(bool zp) { return NS * stage_bytes(zp) + kRS; }

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
  int full;    // workgroups that take a whole 128-row tile; the later ones take 64-row halves
               // (-1: a small call, 64 x 64 pieces only)
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ uint32_t dw4(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

// Byte i of w (two excess-8 nibbles, low = even k) -> two bf16 1 + u/16.
__device__ __forceinline__ uint32_t byte_to_bf16x2(uint32_t w, int i, uint32_t mask, uint32_t one) {
  const uint32_t b = (w >> (8 * i)) & 0xFFu;
  return ((b * 0x8008u) & mask) | one;
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// One output piece of 64 MB rows x 64 NB columns: MB = NB = 2 a whole tile,
// MB = 1 a half (rows 64 sub .. + 64 of its tile), MB = NB = 1 a 64 x 64
// piece of a small call (a.tiles_m and a.tiles_n then count 64-row and
// 64-column pieces).  Wave
// (wm, wn) owns rows 32 MB wm .. + 32 MB and columns 32 NB wn .. + 32 NB
// (blocks of 32 x 32).  qi: the workgroup's index among those of its kind.
// Halves keep their tile's XCD (workgroup id mod 8) under the remap.
template <bool TW, bool ZP, int MB, int NB>
__device__ __forceinline__ void tile_body(const HArgs &a, int qi) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr uint32_t XM = TW ? 0x88888888u : 0u;   // two's complement storage -> excess-8
  constexpr int kStage = stage_bytes(ZP);
  constexpr int NA = 2 * MB;                       // activation loads per wave and step
  constexpr int kVmemPerStep = NA + 1 + 1 + (ZP ? 1 : 0);

  int b = qi, sub = 0;
  if constexpr (MB == 1 && NB == 2) {
    if (a.remap) {
      b = a.full + (qi >> 4) * 8 + (qi & 7);
      sub = (qi >> 3) & 1;
    } else {
      b = a.full + (qi >> 1);
      sub = qi & 1;
    }
  }
  int m_tile, n_tile;
  if (a.remap) {
    const int pn = a.tiles_n >> 3, l = b >> 3;
    n_tile = (b & 7) * pn + l % pn;
    m_tile = l / pn;
  } else {
    m_tile = b % a.tiles_m;
    n_tile = b / a.tiles_m;
  }
  const int m0 = NB == 1 ? m_tile * 64 : m_tile * BM + sub * 64, n0 = n_tile * (64 * NB);
  if (m0 >= a.M) return;   // a half wholly past M (whole workgroup, before any barrier)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;
  const int r32 = lane & 31, hi = lane >> 5;
  const int nsteps = a.K / BK;
  const int spg = a.steps_per_group;

  // ---- staging (rows past M / N clamped) ----
  const __amdgpu_buffer_rsrc_t rs_x = rsrc(a.x, a.M * a.K * 2);
  const __amdgpu_buffer_rsrc_t rs_w = rsrc(a.w, a.N * a.Kb);
  const __amdgpu_buffer_rsrc_t rs_s = rsrc(a.s, a.N * a.Gn * 2);
  const __amdgpu_buffer_rsrc_t rs_z = rsrc(a.z, ZP ? a.N * a.Gn : 0);
  // activations: wave wv, load j writes LDS rows 8 (NA wv + j) .. + 8; lane
  // i lands at row + i / 8, position i % 8, and so loads chunk (i % 8) ^ f(row)
  int a_voff[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = 8 * (NA * wv + j) + (lane >> 3);
    a_voff[j] = min(m0 + r, a.M - 1) * (a.K * 2) + (((lane & 7) ^ swz8(r)) << 4);
  }
  // weights: wave wv writes weight rows 32 bw .. + 32 (32 bytes each); with
  // 64 columns waves 2 and 3 write the same bytes as waves 0 and 1
  const int bw = NB == 2 ? wv : (wv & 1);
  const int b_voff = min(n0 + 32 * bw + (lane >> 1), a.N - 1) * a.Kb + (lane & 1) * 16;
  // scales and zero points: lane i of wave wv takes column 32 NB wn + i
  // (with 64 columns, i mod 32)
  const int scol = min(n0 + 32 * NB * wn + (NB == 2 ? lane : (lane & 31)), a.N - 1);
  const int s_voff = scol * a.Gn * 2;
  const int z_voff = scol * a.Gn;
  const uint32_t smem_lds = lds_addr(smem);

  // ig, ic: group of the next step to request and its place in the group
  // (counted, not divided: the step loop needs no integer division)
  int ig = 0, ic = 0;
  auto issue = [&](auto stage_c, int s) {
    constexpr int S = decltype(stage_c)::value;
    s = min(s, nsteps - 1);
    // the clamped re-reads of the last step take its group
    const int g = __builtin_amdgcn_readfirstlane(min(ig, a.Gn - 1));
    if (++ic == spg) {
      ic = 0;
      ++ig;
    }
    const uint32_t st = smem_lds + S * kStage;
#pragma unroll
    for (int j = 0; j < NA; ++j) dma16(rs_x, st + (NA * wv + j) * 1024, a_voff[j], s * (BK * 2));
    dma16(rs_w, st + kA + bw * 1024, b_voff, s * (BK / 2));
    dma2(rs_s, st + kA + kB + wv * 256, s_voff, g * 2);
    if constexpr (ZP) dma1(rs_z, st + kA + kB + kS + wv * 256, z_voff, g);
  };

  // ---- fragment addresses (stage-relative) ----
  // The lane's activation rows are 32 MB wm + 32 mb + r32, whose chunk
  // swizzle depends on r32 mod 16 only.  a_off[j]: slice j of block 0 (block
  // 1 is 32 rows, 4096 bytes, further on).
  const int fa = swz8(r32);
  int a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) a_off[j] = (32 * MB * wm + r32) * 128 + (((4 * hi + j) ^ fa) << 4);
  const int b_off = kA + (32 * NB * wn + r32) * 32 + hi * 16;   // block nb: + 32 nb * 32
  float *rsum = reinterpret_cast<float *>(smem + NS * kStage) + wv * 64;   // [MB][32]

  f32x16 acc[MB][NB];
  float t[MB][NB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[mb][nb] = f32x16{};
#pragma unroll
      for (int r = 0; r < 16; ++r) t[mb][nb][r] = 0.0f;
    }
  // this lane's half-row sums of x over the group (row r32 of each block),
  // one chain per k slice so that the sums do not wait on each other
  float xs[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) xs[mb][j] = 0.0f;

  uint32_t mask = 0x00780078u, one = 0x3F803F80u;
  asm("" : "+v"(mask), "+v"(one));

  // one K step on stage S; FIRST: the step opens a group
  auto compute = [&](auto stage_c, auto first_c) {
    constexpr int S = decltype(stage_c)::value;
    constexpr bool FIRST = decltype(first_c)::value;
    const uint8_t *st = smem + S * kStage;
    uint4 raw[NB], af[MB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) raw[nb] = *reinterpret_cast<const uint4 *>(st + b_off + nb * 1024);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) af[mb][j] = *reinterpret_cast<const uint4 *>(st + a_off[j] + mb * 4096);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 bq[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t w = dw4(raw[nb], j) ^ XM;
        bq[nb] = make_uint4(byte_to_bf16x2(w, 0, mask, one), byte_to_bf16x2(w, 1, mask, one),
                            byte_to_bf16x2(w, 2, mask, one), byte_to_bf16x2(w, 3, mask, one));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = mfma_bf16_32x32x16(af[mb][j], bq[nb], (FIRST && j == 0) ? f32x16{} : acc[mb][nb]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float v = xs[mb][j];
#pragma unroll
        for (int d = 0; d < 4; ++d) v = dot2_bf16(dw4(af[mb][j], d), 0x3F803F80u, v);
        xs[mb][j] = v;
      }
    }
  };

  // end of a group on stage S: t += 16 s (D - 1.5 sum x), or with zero
  // points t += 16 s (D - (1 + z/16) sum x)
  auto fold = [&](auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    const uint8_t *st = smem + S * kStage;
    // whole-row sums (the two lane halves), into the wave's LDS area
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const float v = add_xor32((xs[mb][0] + xs[mb][1]) + (xs[mb][2] + xs[mb][3]));
      if (hi == 0) rsum[mb * 32 + r32] = v;
#pragma unroll
      for (int j = 0; j < 4; ++j) xs[mb][j] = 0.0f;
    }
    float sc[NB], cb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t sv = *reinterpret_cast<const uint32_t *>(st + kA + kB + wv * 256 + (32 * nb + r32) * 4);
      sc[nb] = 16.0f * bf16_to_f32(sv & 0xFFFFu);
      if constexpr (ZP) {
        const uint32_t zv = *reinterpret_cast<const uint32_t *>(st + kA + kB + kS + wv * 256 + (32 * nb + r32) * 4);
        cb[nb] = -(1.0f + static_cast<float>(zv & 0xFFu) * 0.0625f);
      } else {
        cb[nb] = -1.5f;
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float xr[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(rsum + mb * 32 + 8 * q + 4 * hi);
        xr[4 * q] = v.x; xr[4 * q + 1] = v.y; xr[4 * q + 2] = v.z; xr[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float d = fmaf(cb[nb], xr[r], acc[mb][nb][r]);
          t[mb][nb][r] = fmaf(d, sc[nb], t[mb][nb][r]);
        }
    }
  };

  int cs = 0;   // the computed step's place in its group
  auto step = [&](auto stage_c, int s) {
    constexpr int S = decltype(stage_c)::value;
    wait_vmcnt<kVmemPerStep>();   // this wave's loads of step s are complete
    lds_barrier();                // every wave's are; stage (s + 2) % NS is free
    issue(std::integral_constant<int, (S + 2) % NS>{}, s + 2);
    if (cs == 0) compute(stage_c, std::true_type{});
    else compute(stage_c, std::false_type{});
    if (++cs == spg) {
      cs = 0;
      fold(stage_c);
    }
  };

  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);
  int s = 0;
  for (; s + 2 < nsteps; s += 3) {
    step(std::integral_constant<int, 0>{}, s);
    step(std::integral_constant<int, 1>{}, s + 1);
    step(std::integral_constant<int, 2>{}, s + 2);
  }
  if (s < nsteps) step(std::integral_constant<int, 0>{}, s);
  if (s + 1 < nsteps) step(std::integral_constant<int, 1>{}, s + 1);
  // the ring's last requests (clamped re-reads) must land before the
  // workgroup ends and its LDS is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- output ----
  const int mrow0 = m0 + wm * 32 * MB, ncol0 = n0 + wn * 32 * NB;
  const int64_t rem = static_cast<int64_t>(a.M - mrow0) * a.N - ncol0;
  const int64_t nel = rem > 0 ? min(rem, static_cast<int64_t>(32 * MB) * a.N) : 0;
  const size_t base = rem > 0 ? static_cast<size_t>(mrow0) * a.N + ncol0 : 0;
  const __amdgpu_buffer_rsrc_t rs_yf = rsrc(a.yf ? a.yf + base : nullptr, a.yf ? static_cast<int>(nel * 4) : 0);
  const __amdgpu_buffer_rsrc_t rs_yb = rsrc(a.yb ? a.yb + base : nullptr, a.yb ? static_cast<int>(nel * 2) : 0);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int col = nb * 32 + r32;
    const bool col_ok = ncol0 + col < a.N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * mb + 8 * (r >> 2) + 4 * hi + (r & 3);
        const int e = col_ok ? row * a.N + col : (1 << 28);
        const float v = t[mb][nb][r];
        if (a.yf) __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs_yf, e * 4, 0, kStoreStream);
        if (a.yb) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), rs_yb, e * 2, 0, kStoreStream);
      }
  }
}

// One launch per call: the first a.full workgroups take whole tiles, the
// rest the 64-row halves of the other tiles.
template <bool TW, bool ZP>
__global__ __launch_bounds__(kThreads, 2) void tiled_w4a16_kernel(HArgs a) {
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < a.full) tile_body<TW, ZP, 2, 2>(a, bid);
  else tile_body<TW, ZP, 1, 2>(a, bid - a.full);
}

// Small calls (at most 64 rows, or pieces that fit one round of
// workgroups): one 64 x 64 piece per workgroup, four per tile.
template <bool TW, bool ZP>
__global__ __launch_bounds__(kThreads, 2) void tiled_w4a16_small(HArgs a) {
  tile_body<TW, ZP, 1, 1>(a, static_cast<int>(blockIdx.x));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <bool TW, bool ZP>
hipError_t launch_k(const HArgs &a, hipStream_t st) {
  // more than 64 KB of dynamic LDS per workgroup must be allowed explicitly
  static const bool attr =
      hipFuncSetAttribute(reinterpret_cast<const void *>(tiled_w4a16_kernel<TW, ZP>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes(ZP)) == hipSuccess &&
      hipFuncSetAttribute(reinterpret_cast<const void *>(tiled_w4a16_small<TW, ZP>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes(ZP)) == hipSuccess;
  if (!attr) return hipErrorInvalidValue;
  if (a.full < 0) {   // one 64 x 64 piece per workgroup
    const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.tiles_m) * a.tiles_n);
    tiled_w4a16_small<TW, ZP><<<dim3(grid), kThreads, lds_bytes(ZP), st>>>(a);
    return hipGetLastError();
  }
  // whole tiles, then the halves, in one grid
  const int64_t tiles = static_cast<int64_t>(a.tiles_m) * a.tiles_n;
  const dim3 grid(static_cast<unsigned>(a.full + (tiles - a.full) * 2));
  tiled_w4a16_kernel<TW, ZP><<<grid, kThreads, lds_bytes(ZP), st>>>(a);
  return hipGetLastError();
}

}  // namespace

bool tiled_w4a16_ok(const void *x, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G) {
  if (M < 17 || K <= 0 || K % BK != 0 || G <= 0 || G % BK != 0 || K % G != 0) return false;
  if (!aligned16(x) || !aligned16(wq)) return false;
  if (M * K * 2 >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31)) return false;
  if (N * (K / G) * 2 >= (int64_t(1) << 31)) return false;
  if (256 * N >= (int64_t(1) << 29)) return false;   // byte offsets within 64 rows stay below 2^29
  return true;
}

// Work split of one call: `full` whole 128 x 128 tiles first, then the
// other tiles cut into two 64-row halves (the same launch); `pieces` counts
// the workgroups of 64 rows.  Small calls, at most 64 rows or so few tiles
// that four 64 x 64 pieces per tile fit one round of workgroups (two per
// CU), run as such pieces only (full = -1).  Otherwise the tiles past the
// last whole round are cut when their halves fit one round.  Halves keep
// the XCD grouping by eights, so the cut is dropped when the cut tiles do
// not come in eights.
void tiled_w4a16_pieces(int64_t M, int64_t N, int cus, int *full, int64_t *pieces) {
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = ((M + BM - 1) / BM) * tiles_n;
  const int64_t slots = 2 * static_cast<int64_t>(cus);
  if (M <= 64 || tiles * 4 <= slots) {
    *full = -1;
    *pieces = ((M + 63) / 64) * ((N + 63) / 64);
    return;
  }
  const bool remap = tiles_n % 8 == 0;
  const int64_t rem = slots > 0 ? tiles % slots : 0;
  *full = static_cast<int>(tiles);
  if (remap && slots > 0 && tiles >= slots && rem > 0 && rem * 2 <= slots) *full = static_cast<int>(tiles - rem);
  if (remap && (tiles - *full) % 8 != 0) *full = static_cast<int>(tiles);
  *pieces = (tiles - *full) * 2;
}

hipError_t launch_tiled_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf, uint16_t *yb,
                              int64_t M, int64_t N, int64_t K, int64_t G, int enc, hipStream_t st,
                              const uint8_t *zp) {
  HArgs a{};
  a.x = x; a.w = wq; a.s = s; a.yf = yf; a.yb = yb; a.z = zp;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(K / 2);
  a.Gn = static_cast<int>(K / G);
  a.steps_per_group = static_cast<int>(G / BK);
  int64_t pieces = 0;
  tiled_w4a16_pieces(M, N, device_cu_count(), &a.full, &pieces);
  const int64_t unit = a.full < 0 ? 64 : BM;   // 64 x 64 pieces, or 128 x 128 tiles
  a.tiles_m = static_cast<int>((M + unit - 1) / unit);
  a.tiles_n = static_cast<int>((N + unit - 1) / unit);
  a.remap = (a.tiles_n % 8 == 0) ? 1 : 0;
  if (zp) return launch_k<false, true>(a, st);   // zero points: the stored u as is
  if (enc == kTwos) return launch_k<true, false>(a, st);
  return launch_k<false, false>(a, st);
}

}  // namespace q4
