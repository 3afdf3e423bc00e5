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
//   * Workgroup tile 128 x 128 of y, K in steps of 128 (one weight group per
//     step in the grouped form), two workgroups per CU.  Wave w owns the 32
//     output columns 32w..32w+31 and all 128 rows: four 32 x 32 blocks on
//     v_mfma_i32_32x32x32_i8 (the full-rate int8 shape).
//   * Staging: the activation tile (128 rows x 128 int8) and the packed
//     weight tile (128 rows x 64 bytes) go from global memory straight into
//     LDS with buffer loads that write LDS (16 bytes per lane, lane i at
//     base + 16 i), into a ring of three stages, issued two steps ahead; the
//     group scales travel the same way, and so do the zero points (a byte
//     per lane).  (A zero point loaded into a register instead made every
//     step wait for the next two steps' staging loads: the compiler counts
//     its own loads only, and loads complete in order.)  No registers hold staged data, and
//     a step waits only for loads issued two steps earlier.  One barrier per
//     step.
//   * LDS layout: the 16-byte chunk c of activation row r (128 bytes) sits at
//     position c ^ f(r), and chunk c of weight row r (64 bytes) at
//     c ^ g(r); a lane's load address picks the chunk that belongs at its
//     slot.  f and g make every 8- and 16-lane phase of the fragment reads
//     touch distinct banks.
//   * Weights are unpacked in registers by the wave that uses them (each
//     column by exactly one wave): one 16-byte LDS read per lane holds the
//     32 codes of k = 64P + 32h + 0..31 for its column (h = lane / 32), which
//     become the B operands of two MFMAs (k + 0..15 and k + 16..31).  The A
//     operand of lane (row, h) is then the 16-byte activation chunk with the
//     same k, so each MFMA sums 32 distinct k and the four MFMAs of a block
//     cover the 128 k of the step exactly once (the integer sum does not
//     depend on the order).
//   * A nibble is moved to the top half of its byte, where the
//     two's-complement code q reads as the int8 16*q (a shift, two masks and
//     two byte permutes per 8 nibbles); no +8 bias is left to cancel and the
//     MFMA sums are exactly 16*acc.  With per-group zero points z ("The 4-bit
//     CPU path", section W4A8: they take the place of the constant 8) the
//     bytes are u - z instead, as ((u + (0x80 - z)) ^ 0x80) per byte (u +
//     0x80 - z lies in 113..143, so no carry crosses a byte), and the sums
//     are acc itself.
//   * Per channel f32(16*acc) * 2^-4 = f32(acc) exactly, then the two scale
//     multiplies.
//   * Grouped: each group's MFMA sum starts from the bits of c = 1.5 * 2^19
//     (0x49400000; 1.5 * 2^23 = 0x4B400000 with zero points) instead of 0.
//     c's mantissa field is 2^22, and |16*acc_g| <= 128*127*128 = 2080768
//     (|acc_g| <= 128*127*15 with zero points) is less than both 2^22 and
//     its distance to 2^23, so the i32 sum's bits are the float
//     F = c + acc_g exactly: the sum moves c's mantissa by 16*acc_g units of
//     2^-4 (by acc_g units of 1), inside c's binade.  F - c = f32(acc_g) is
//     exact, and (F - c) * s_g is the product of the plain form for every
//     scale: a subtraction where an integer-to-float conversion would take
//     a slower instruction.  Then t = t + p; t starts at -0.0, the identity
//     of f32 addition.
//   * Fast form of that epilogue: when c * s_g is exact (c = 1.5 * 2^k, so
//     whenever 3 s_g is: every bf16 or f16 value) and s_g > 0,
//     fma(F, s_g, -(c s_g)) = (c + acc_g) s_g - c s_g is acc_g s_g rounded
//     once, the same product, in one instruction instead of two; an exact
//     zero product keeps the sign +0 of f32(acc_g) * s_g.  Each wave checks
//     every scale of its 32 columns before its first step (they are one
//     contiguous run of the scale matrix, staged like the tiles) and runs
//     the whole tile in the fast form if all pass, else in the plain form.
//     On this chip the MFMAs and the epilogue's VALU work hardly overlap, so
//     the epilogue's instruction count is a large share of the time.
//   * The MFMAs of a step run block by block, and the epilogue of block b
//     (its 16 outputs per lane: subtract, multiply, add) is issued among the
//     MFMAs of block b + 1; the last block's epilogue runs among the next
//     step's first MFMAs.  The two workgroups on a CU fill each other's
//     waits.
//   * Tiles are ordered so that each XCD (workgroup id mod 8) owns a band of
//     weight columns and walks all activation rows: its weights stay in its
//     L2 while the activation tiles stream through.
#include <atomic>
#include <type_traits>

#include "kernels.hpp"
#include "q4_device.hpp"
#include "q4_lds_dma.hpp"

namespace q4 {
namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int NS = 3;                         // LDS ring stages
constexpr int kA = BM * BK;                   // activation tile, int8 (16 KB)
constexpr int kB = BN * BK / 2;               // packed weight tile (8 KB)
constexpr int kS = 4 * 64 * 4;                // group scales, 4 waves x 64 lanes x 4 bytes
constexpr int kZ = 4 * 64 * 4;                // zero points (ZP kernels): one byte per lane in a 4-byte slot
constexpr int stage_bytes(bool zp) { return kA + kB + kS + (zp ? kZ : 0); }
constexpr int lds_bytes(bool zp) { return NS * stage_bytes(zp) + (BM + BN) * 4; }

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
  int full;        // workgroups that take a whole 128-row tile
  int split;       // later workgroups take 1/split of a tile's rows (1, 2 or 4)
  const uint8_t *z;  // per-group zero points [N, K/G] (ZP kernel only)
  int sw_al16;       // scales 16-byte aligned (the fast-form check reads them 16 bytes at a time)
};

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// Cache policy of the output stores (sc0 | nt): y is written once and not
// read back, so it streams past the caches instead of displacing the tiles
// other workgroups still read (measured: 3-4% faster at the prefill shape).
constexpr int kStoreStream = 3;

// Start value of a grouped MFMA sum, as bits of a binary32: 1.5 * 2^19 when
// the sum counts 16 acc (units 2^-4), 1.5 * 2^23 when it counts acc.
constexpr int kSumStart16 = 0x49400000;
constexpr int kSumStart1 = 0x4B400000;

// Chunk position permutations (activation rows: 8 chunks; weight rows: 4).
__device__ __forceinline__ int swz_a(int r) { return swz8(r); }
__device__ __forceinline__ int swz_b(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }

__device__ __forceinline__ i32x16 mfma_i8_32x32x32(uint4 a, uint4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0,
                                               0, 0);
}


// 8 nibbles (k0..k7 of one packed dword) -> 8 signed bytes in k order:
// 16*q (zero point absent) or u - z (cz = (0x80 - z) in every byte).
template <bool ZP, uint32_t XM>
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t cz, uint32_t &o0, uint32_t &o1) {
  uint32_t lo, hi;
  if constexpr (ZP) {
    lo = ((w & 0x0F0F0F0Fu) + cz) ^ 0x80808080u;
    hi = (((w >> 4) & 0x0F0F0F0Fu) + cz) ^ 0x80808080u;
  } else {
    if constexpr (XM != 0u) {
      // excess-8 to two's complement first, as a plain XOR: folded into
      // the masks below it would become a three-input bit operation, which
      // issues more slowly here
      asm("v_xor_b32 %0, %1, %2" : "=v"(w) : "v"(w), "s"(XM));
    }
    lo = (w << 4) & 0xF0F0F0F0u;
    hi = w & 0xF0F0F0F0u;
  }
  o0 = perm_b32(hi, lo, 0x05010400u);   // k0..k3
  o1 = perm_b32(hi, lo, 0x07030602u);   // k4..k7
}

// Workgroup -> tile.  Tiles are ordered so that each XCD (workgroup id mod 8)
// owns a band of weight columns and walks all activation rows: its weights
// stay in its L2 while the activation tiles stream through.  The kernel with
// NMB = 4 takes the first a.full tiles whole; the kernels with NMB = 2 or 1
// take the rest in sub-tiles of 32 NMB rows, which keep the XCD of their
// whole tile (this fills the last, partial round of workgroups with short
// ones, and serves small M without computing rows past it).
// Each workgroup computes one output tile of 32 NMB rows x 128 columns: NMB
// blocks of 32 rows per wave.
// qi: the workgroup's index among those of its NMB.
template <bool GROUPED, bool TW, bool ZP, int NMB>
__device__ __forceinline__ void tile_body(const TArgs &a, int qi) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int nsub = 4 / NMB;
  int b = qi, sub = 0;
  if constexpr (nsub > 1) {
    if (a.remap) {
      b = a.full + (qi / (8 * nsub)) * 8 + (qi & 7);
      sub = (qi >> 3) % nsub;
    } else {
      b = a.full + qi / nsub;
      sub = qi % nsub;
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
  const int m0 = m_tile * BM + sub * (32 * NMB), n0 = n_tile * BN;
  if (m0 >= a.M) return;   // a sub-tile wholly past M (whole workgroup, before any barrier)

  static_assert(!ZP || (GROUPED && !TW), "zero points: grouped, stored nibbles used as is");
  constexpr int kStage = stage_bytes(ZP);
  static_assert(NMB == 1 || NMB == 2 || NMB == 4, "row blocks per tile");
  // excess-8 storage becomes two's complement under u ^ 8
  constexpr uint32_t XM = TW ? 0u : 0x88888888u;
  // loads per wave and step: NMB activation, 2 weight, 1 scale (grouped), 1 zero point
  constexpr int kVmemPerStep = NMB + 2 + (GROUPED ? 1 : 0) + (ZP ? 1 : 0);
  float *Sx = reinterpret_cast<float *>(smem + NS * kStage);   // [BM]
  float *Sw = Sx + BM;                                           // [BN] per-channel scales

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;

  const int nsteps = a.K / BK;


  // ---- staging: global -> LDS (rows past M / N clamped) ----
  const __amdgpu_buffer_rsrc_t rs_a = rsrc(a.xq, a.M * a.K);
  const __amdgpu_buffer_rsrc_t rs_b = rsrc(a.w, a.N * a.Kb);
  // Activations: wave wv, load j writes LDS rows 8 (NMB wv + j) .. + 8; lane
  // i lands at row + i / 8, position i % 8 and so loads chunk (i % 8) ^ f(row).
  int a_voff[NMB];
#pragma unroll
  for (int j = 0; j < NMB; ++j) {
    const int r = 8 * (NMB * wv + j) + (lane >> 3);
    a_voff[j] = min(m0 + r, a.M - 1) * a.K + (((lane & 7) ^ swz_a(r)) << 4);
  }
  // Weights: wave wv, load j writes LDS rows 16 (2 wv + j) .. + 16 of 64
  // bytes; lane i lands at row + i / 4, position i % 4.
  int b_voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * (2 * wv + j) + (lane >> 2);
    b_voff[j] = min(n0 + r, a.N - 1) * a.Kb + (((lane & 3) ^ swz_b(r)) << 4);
  }
  // this lane's output column and, grouped, its scale (and zero point) row
  const int col = 32 * wv + l32;
  const int ncl = min(n0 + col, a.N - 1);
  const __amdgpu_buffer_rsrc_t rs_s = rsrc(a.sw, GROUPED ? a.N * a.Gn * 4 : 4);
  const __amdgpu_buffer_rsrc_t rs_z = rsrc(a.z, ZP ? a.N * a.Gn : 0);
  const int s_voff = GROUPED ? ncl * a.Gn * 4 : 0;   // lanes l and l + 32 load the same scale
  const int z_voff = ZP ? ncl * a.Gn : 0;
  const uint32_t smem_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)smem));

  constexpr int kSumStart = ZP ? kSumStart1 : kSumStart16;

  // loads of step s (clamped to the last step, whose data an idle stage may
  // receive again) into stage S = s % NS
  auto issue = [&](auto stage_c, int s) {
    constexpr int S = decltype(stage_c)::value;
    s = min(s, nsteps - 1);
    const uint32_t st = smem_lds + S * kStage;
#pragma unroll
    for (int j = 0; j < NMB; ++j) dma16(rs_a, st + (NMB * wv + j) * 1024, a_voff[j], s * BK);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(rs_b, st + kA + (2 * wv + j) * 1024, b_voff[j], s * (BK / 2));
    if constexpr (GROUPED) dma4(rs_s, st + kA + kB + wv * 256, s_voff, s * 4);
    if constexpr (ZP) dma1(rs_z, st + kA + kB + kS + wv * 256, z_voff, s);
  };

  // ---- fragment addresses (stage-relative) ----
  // Weights: lane (col, h) reads chunk 2P + h of its column's row.
  const int b_off0 = kA + col * 64 + (((0 + lh) ^ swz_b(col)) << 4);
  const int b_off1 = kA + col * 64 + (((2 + lh) ^ swz_b(col)) << 4);
  // Activations: lane (r, h) of block mb reads chunk 4P + 2h + j of row
  // 32 mb + r (swz_a depends on the row mod 16 only).
  const int fa = swz_a(l32);
  int a_off[4];                // index 2P + j
#pragma unroll
  for (int pj = 0; pj < 4; ++pj) {
    const int c = 4 * (pj >> 1) + 2 * lh + (pj & 1);
    a_off[pj] = l32 * 128 + ((c ^ fa) << 4);
  }

  // acc[mb]: block mb of the wave's 32 NMB x 32 tile; register r of lane l
  // holds row 32 mb + 8 (r / 4) + 4 (l / 32) + r % 4, column 32 wv + l % 32.
  i32x16 acc[NMB];
  float t[NMB][16];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[mb][r] = 0;
      t[mb][r] = -0.0f;
    }

  // Grouped epilogue of block mb: t += f32(acc_g) * s_g, where the sums
  // hold F = c + acc_g (c = 1.5 * 2^k).
  //   fast form: when c * s_g is exact (whenever 3 s_g is, which every bf16
  //     or f16 value is) and s_g > 0, fma(F, s_g, -(c s_g)) = (c + acc_g)
  //     s_g - c s_g = acc_g s_g rounded once, the product itself, and an
  //     exact zero product gets the sign +0 that f32(acc_g) * s_g has; then
  //     the add.  Two instructions per sum.
  //   plain form: F - c = f32(acc_g), the multiply, the add.
  // A wave runs the whole tile in one form: the fast one when every scale
  // of its columns passes the check (below).  Each pass runs over all 16
  // sums in place, so its instructions do not wait on each other.
  const float cst = __int_as_float(kSumStart);
  auto epi = [&](auto fast_c, int mb, float sg, float csg) {
    if constexpr (decltype(fast_c)::value) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        acc[mb][r] = __float_as_int(__builtin_fmaf(__int_as_float(acc[mb][r]), sg, csg));
    } else {
      (void)csg;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = __float_as_int(__int_as_float(acc[mb][r]) - cst);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][r] = __float_as_int(__int_as_float(acc[mb][r]) * sg);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) t[mb][r] = t[mb][r] + __int_as_float(acc[mb][r]);
  };

  // The last block's epilogue of a step is carried into the next step.  The
  // first step carries an identity: a sum equal to the start value with
  // scale -0.0 gives p = (c - c) * -0.0 = -0.0 (fast form: fma(c, -0.0,
  // -0.0) = -0.0), and -0.0 + -0.0 leaves t at -0.0.
  float pend_s = -0.0f, pend_cs = -0.0f;
  if constexpr (GROUPED) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[NMB - 1][r] = kSumStart;
  }

  // One K step on stage S: block by block, the next block's activation
  // fragments are read while the current block's MFMAs run, with the
  // previous block's epilogue (block 0: the previous step's block 3) among
  // them.
  auto mma = [&](auto fast_c, auto stage_c, const uint4 (&bop)[2][2], const uint4 (&af0)[4], float sg, float csg) {
    constexpr int S = decltype(stage_c)::value;
    const uint8_t *st = smem + S * kStage;
    uint4 af[2][4];
#pragma unroll
    for (int pj = 0; pj < 4; ++pj) af[0][pj] = af0[pj];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if (mb < NMB - 1) {
        const uint8_t *ar = st + (mb + 1) * 32 * 128;
#pragma unroll
        for (int pj = 0; pj < 4; ++pj) af[(mb + 1) & 1][pj] = *reinterpret_cast<const uint4 *>(ar + a_off[pj]);
      }
      // with a single block, the carried epilogue reads the sums this
      // step's MFMAs replace, so it goes first
      if constexpr (GROUPED && NMB == 1) epi(fast_c, 0, pend_s, pend_cs);
      // the next block's reads stay here, ahead of this block's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pj = 0; pj < 4; ++pj) {
        const i32x16 start = {kSumStart, kSumStart, kSumStart, kSumStart, kSumStart, kSumStart,
                              kSumStart, kSumStart, kSumStart, kSumStart, kSumStart, kSumStart,
                              kSumStart, kSumStart, kSumStart, kSumStart};
        // (mutant s04: a group's sum continues from the previous group's)
        const i32x16 c0 = (GROUPED && pj == 0 && Q4_MUTANT != 4) ? start : acc[mb];
        acc[mb] = mfma_i8_32x32x32(af[mb & 1][pj], bop[pj >> 1][pj & 1], c0);
      }
      if constexpr (GROUPED) {
        if (mb > 0) epi(fast_c, mb - 1, sg, csg);
        else if (NMB > 1) epi(fast_c, NMB - 1, pend_s, pend_cs);
        // each MFMA followed by a quarter of the previous block's epilogue
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (GROUPED) {
      pend_s = sg;
      pend_cs = csg;
    }
  };

  auto step = [&](auto fast_c, auto stage_c, int s) {
    constexpr int S = decltype(stage_c)::value;
    // this wave's loads of step s are complete once only step s + 1's remain
    wait_vmcnt<kVmemPerStep>();
    lds_barrier();   // every wave's loads of step s landed; stage (s + 2) % NS is free
    issue(std::integral_constant<int, (S + 2) % NS>{}, s + 2);
    const uint8_t *st = smem + S * kStage;

    // the B operands of the step (k = 64P + 32h + 16j + 0..15) and the
    // first block's activation fragments: the unpack covers the reads
    const uint4 raw0 = *reinterpret_cast<const uint4 *>(st + b_off0);
    const uint4 raw1 = *reinterpret_cast<const uint4 *>(st + b_off1);
    uint4 af0[4];
#pragma unroll
    for (int pj = 0; pj < 4; ++pj) af0[pj] = *reinterpret_cast<const uint4 *>(st + a_off[pj]);
    uint4 bop[2][2];
    uint32_t cz = 0u;
    if constexpr (ZP) cz = (0x80u - (*reinterpret_cast<const uint32_t *>(st + kA + kB + kS + wv * 256 + lane * 4) & 0xFFu)) * 0x01010101u;
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const uint4 raw = P ? raw1 : raw0;
      uint32_t o[8];
      unpack8<ZP, XM>(raw.x, cz, o[0], o[1]);
      unpack8<ZP, XM>(raw.y, cz, o[2], o[3]);
      unpack8<ZP, XM>(raw.z, cz, o[4], o[5]);
      unpack8<ZP, XM>(raw.w, cz, o[6], o[7]);
      bop[P][0] = make_uint4(o[0], o[1], o[2], o[3]);
      bop[P][1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
    float sg = 0.0f, csg = 0.0f;
    if constexpr (GROUPED) sg = *reinterpret_cast<const float *>(st + kA + kB + wv * 256 + l32 * 4);
    if constexpr (decltype(fast_c)::value) csg = -(cst * sg);
    mma(fast_c, stage_c, bop, af0, sg, csg);
  };

  // ---- main loop: one barrier per step, unrolled by the ring size ----
  // Grouped: the check of the fast form (s > 0, c * s finite and exact)
  // over every scale of the wave's 32 columns, which are one contiguous run
  // of 128 Gn bytes of the scale matrix.  The run goes into the third ring
  // stage (idle until the first step stages step 2 there), 1 KB per load
  // that writes LDS, up to 4 KB per wave at a time; the first loads are
  // requested before the first two steps' loads, so the wait covers them
  // only.  Each lane checks the 16 bytes its own load wrote.  Scales that
  // are not 16-byte aligned take the plain form without a check.
  // Row scales (waves 0 and 1) and, per channel, column scales (waves 2 and
  // 3) go to LDS by loads that write LDS, ahead of every staging load: the
  // output alone needs them, and a load into a register made each tile
  // start wait for it before its staging loads were requested.
  {
    const uint32_t sxw = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)Sx));
    if (wv < 2) {
      dma4(rsrc(a.sx, a.M * 4), sxw + wv * 256, min(m0 + 64 * wv + lane, a.M - 1) * 4, 0);
    } else if constexpr (!GROUPED) {
      dma4(rsrc(a.sw, a.N * 4), sxw + BM * 4 + (wv - 2) * 256, min(n0 + 64 * (wv - 2) + lane, a.N - 1) * 4, 0);
    }
  }

  bool fast = false;
  if constexpr (GROUPED) {
    const int wc0 = min(n0 + 32 * wv, a.N), wc1 = min(n0 + 32 * wv + 32, a.N);
    const int rbeg = wc0 * a.Gn * 4, nbytes = a.sw_al16 ? (wc1 - wc0) * a.Gn * 4 : 0;
    const uint32_t chk = smem_lds + 2 * kStage + wv * 4096;
    const uint8_t *chk_p = smem + 2 * kStage + wv * 4096 + lane * 16;
    bool ok = nbytes > 0;
    for (int c0 = 0; c0 < nbytes || c0 == 0; c0 += 4096) {
      const int nch = min(4, (nbytes - c0 + 1023) >> 10);
      for (int j = 0; j < nch; ++j) dma16(rs_s, chk + j * 1024, lane * 16, rbeg + c0 + j * 1024);
      if (c0 == 0) {
        issue(std::integral_constant<int, 0>{}, 0);
        issue(std::integral_constant<int, 1>{}, 1);
        wait_vmcnt<2 * kVmemPerStep>();
      } else {
        wait_vmcnt<0>();
      }
      for (int j = 0; j < nch; ++j) {
        const uint4 v = *reinterpret_cast<const uint4 *>(chk_p + j * 1024);   // after the wait (a memory clobber)
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sv = __uint_as_float(w4[e]);
          const float cs = cst * sv;
          const bool pass = (sv > 0.0f) & (cs <= 3.402823466e38f) & (__builtin_fmaf(cst, sv, -cs) == 0.0f);
          ok = ok & (pass | (c0 + j * 1024 + lane * 16 + 4 * e >= nbytes));
        }
      }
    }
    fast = __builtin_amdgcn_ballot_w64(!ok) == 0;   // uniform over the wave
  } else {
    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
  }
  auto main_loop = [&](auto fast_c) {
    for (int s = 0; s < nsteps; s += NS) {
      step(fast_c, std::integral_constant<int, 0>{}, s);
      if (s + 1 < nsteps) step(fast_c, std::integral_constant<int, 1>{}, s + 1);
      if (s + 2 < nsteps) step(fast_c, std::integral_constant<int, 2>{}, s + 2);
    }
    if constexpr (GROUPED) epi(fast_c, NMB - 1, pend_s, pend_cs);
  };
  // both forms pass the same barriers
  if (fast) main_loop(std::true_type{});
  else main_loop(std::false_type{});
  wait_vmcnt<0>();   // the last steps' reloads of idle stages

  // ---- output: y = t * sx (grouped) or ((f32(16 acc) / 16) * sx) * sw ----
  // Stores go through a buffer whose bounds end at y[M-1][N-1] (counted from
  // this tile's first element): rows past M fall outside it, columns past N
  // get an offset far outside it, and the hardware drops those stores.
  const int64_t rem = static_cast<int64_t>(a.M - m0) * a.N - n0;
  const int nrec = rem > 0 ? static_cast<int>(min(rem, static_cast<int64_t>(32 * NMB) * a.N) * 4) : 0;
  const __amdgpu_buffer_rsrc_t rs_y = rsrc(a.y + (rem > 0 ? static_cast<size_t>(m0) * a.N + n0 : 0), nrec);
  const int vcol = (n0 + col < a.N) ? col * 4 : (1 << 30);
  const float swc = GROUPED ? 0.0f : Sw[col];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rl = mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);   // tile-relative row
      const float sxr = Sx[rl];
      float v;
      if constexpr (GROUPED) {
        v = t[mb][r] * sxr;
      } else {
        const float f = static_cast<float>(acc[mb][r]) * 0.0625f;
        v = (f * sxr) * swc;
      }
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs_y, rl * a.N * 4 + vcol, 0, kStoreStream);
    }
  }
}


// One launch per call: the first a.full workgroups take whole tiles, the
// rest the sub-tiles of 32 * 4 / split rows, so the sub-tiles start in the
// slots the last whole tiles free, with no kernel boundary between.
template <bool GROUPED, bool TW, bool ZP>
__global__ __launch_bounds__(kThreads, 2) void tiled_w4a8_kernel(TArgs a) {
  const int bid = blockIdx.x;
  if (bid < a.full) tile_body<GROUPED, TW, ZP, 4>(a, bid);
  else if (a.split == 2) tile_body<GROUPED, TW, ZP, 2>(a, bid - a.full);
  else tile_body<GROUPED, TW, ZP, 1>(a, bid - a.full);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }


}  // namespace

// Compute units of the current device (looked up once per device).
int device_cu_count() {
  static std::atomic<int> counts[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = counts[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return 0;
    counts[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

bool tiled_w4a8_ok(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G) {
  if (M < 17 || K <= 0 || K % BK != 0 || !(G == 0 || G == BK)) return false;
  if (!aligned16(xq) || !aligned16(wq)) return false;
  // 32-bit buffer offsets; 16*acc must fit i32 over all of K per channel
  if (M * K >= (int64_t(1) << 31) || N * (K / 2) >= (int64_t(1) << 31)) return false;
  if (G && N * (K / G) * 4 >= (int64_t(1) << 31)) return false;
  if (!G && K > 131072) return false;
  if (BM * 4 * N >= (int64_t(1) << 30)) return false;   // y offsets within a tile stay below 2^30
  return true;
}

// Work split of one call: `full` whole 128-row tiles first, then the other
// tiles cut into `split` pieces of 128 / split rows (the same launch).
// Small calls (at most 64 rows, or so few tiles that their 32-row pieces
// fit one round of workgroups, two per CU): every tile in 32-row pieces
// while all of them fit one round, else in 64-row pieces; pieces past M
// exit at once.  Otherwise the tiles past the last whole round are
// cut into halves when they fill at most half a round.  Sub-tiles keep the
// XCD grouping by eights, so a split is dropped when the cut tiles do not
// come in eights.
void tiled_w4a8_pieces(int64_t M, int64_t N, int cus, int *full, int *split, int64_t *tiles_out) {
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = ((M + BM - 1) / BM) * tiles_n;
  if (tiles_out) *tiles_out = tiles;
  const bool remap = tiles_n % 8 == 0;
  const int64_t slots = 2 * static_cast<int64_t>(cus);
  const int64_t rem = slots > 0 ? tiles % slots : 0;
  *full = static_cast<int>(tiles);
  *split = 1;
  if (M <= 64 || tiles * 4 <= slots) {
    *full = 0;
    *split = tiles * 4 <= slots ? 4 : 2;
  } else if (remap && slots > 0 && tiles >= slots && rem > 0 && rem * 2 <= slots) {
    // halves, not quarters, even where quarters would fill the round: a
    // 32-row piece pays a whole tile's weight unpack and barriers for a
    // quarter of its MFMAs (measured at the prefill shape, 1664 tiles on
    // 512 slots: halves 80-82 us per call, quarters 84-86, no split 82-84)
    *full = static_cast<int>(tiles - rem);
    *split = 2;
  }
  if (remap && *split > 1 && (tiles - *full) % 8 != 0) {
    *full = static_cast<int>(tiles);
    *split = 1;
  }
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
  tiled_w4a8_pieces(M, N, device_cu_count(), &a.full, &a.split, nullptr);
  a.z = zp;
  a.sw_al16 = aligned16(sw) ? 1 : 0;
  static const bool attrs = [] {
    // more than 64 KB of dynamic LDS per workgroup must be allowed explicitly
    bool ok = true;
    auto allow = [&](const void *k, int bytes) {
      ok &= hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    };
    auto all_nmb = [&](auto g_c, auto tw_c, auto zp_c) {
      constexpr bool G = decltype(g_c)::value, T = decltype(tw_c)::value, Z = decltype(zp_c)::value;
      allow(reinterpret_cast<const void *>(tiled_w4a8_kernel<G, T, Z>), lds_bytes(Z));
    };
    all_nmb(std::true_type{}, std::true_type{}, std::false_type{});
    all_nmb(std::true_type{}, std::false_type{}, std::false_type{});
    all_nmb(std::true_type{}, std::false_type{}, std::true_type{});
    all_nmb(std::false_type{}, std::true_type{}, std::false_type{});
    all_nmb(std::false_type{}, std::false_type{}, std::false_type{});
    return ok;
  }();
  if (!attrs) return hipErrorInvalidValue;
  // whole tiles, then the sub-tiles, in one grid
  const unsigned grid = static_cast<unsigned>(a.full + (tiles - a.full) * a.split);
  auto run = [&](auto g_c, auto tw_c, auto zp_c) {
    constexpr bool G = decltype(g_c)::value, T = decltype(tw_c)::value, Z = decltype(zp_c)::value;
    tiled_w4a8_kernel<G, T, Z><<<dim3(grid), kThreads, lds_bytes(Z), st>>>(a);
  };
  if (zp) run(std::true_type{}, std::false_type{}, std::true_type{});
  else if (G && enc == kTwos) run(std::true_type{}, std::true_type{}, std::false_type{});
  else if (G) run(std::true_type{}, std::false_type{}, std::false_type{});
  else if (enc == kTwos) run(std::false_type{}, std::true_type{}, std::false_type{});
  else run(std::false_type{}, std::false_type{}, std::false_type{});
  return hipGetLastError();
}

}  // namespace q4
