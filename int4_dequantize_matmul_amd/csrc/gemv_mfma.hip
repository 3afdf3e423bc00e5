// Decode GEMV on the matrix cores: y[m, n] for up to 16 activation rows.
//
// What it computes (cited by page title and section):
//   W4A16  y = sum_g s[n,g] sum_{k in g} x[m,k] q[n,k]       ("Fused int4 and
//          int8 dequantize-matmul in C", section 2.3), bf16 x and scales,
//          f32 accumulation, bf16 output rounded to nearest even.
//   W4A8   acc = sum_k xq q exactly in i32, the stored +8 bias cancelled by
//          one correction term from the activation sum (ftts_kernels module
//          int4, "Packing" and dot_i32_q4); per channel y = (f32(acc)*sx)*sw,
//          grouped t = f32(acc_0)s_0, t = t + f32(acc_g)s_g in increasing g,
//          y = t*sx (module int8 head: scales once, after accumulation, in a
//          fixed order).
//   W8A8   the same per-channel epilogue with int8 weights.
//
// How (gfx950):
//   * One workgroup of NW waves owns a block of 16 weight rows and 16
//     activation rows.  The K axis is cut into chunks of 64 bytes per row
//     (128 int4 or 64 int8 columns); wave w owns a contiguous run of chunks.
//     Every lane issues all its 16-byte weight loads before touching any of
//     them, so the packed rows stream from HBM once, with many bytes in
//     flight per CU.
//   * MFMA operands: B is the weights (lane 16*q + j holds row j of the
//     block, one 16-byte piece of the chunk), A is the activations (lane
//     16*q + i holds row i of x for the same k slots).  A is loaded straight
//     from global memory into registers (the rows are tiny and stay in L2)
//     and reordered to the k order the unpack produces.
//   * Nibbles are unpacked in registers with shift-and-mask:
//       int8 MFMA: bytes u = w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F;
//       bf16 MFMA: ((w << 3 | w >> 1 | w >> 5 | w >> 9) & 0x00780078) | 0x3F80..
//                  is the exact bf16 value v = 1 + u/16 of each stored u.
//     Two's-complement storage is XORed with 0x88888888 first (t ^ 8 = u).
//   * The stored bias cancels inside the matrix core: a second MFMA with a
//     constant B operand (int8 -8, or bf16 -1.5) adds -8 * sum xq (int8,
//     exact) or -1.5 * sum x (bf16) to the same accumulator, so
//       int8:  D = sum xq u - 8 sum xq      = sum xq q
//       bf16:  D = sum x v - 1.5 sum x      = (1/16) sum x q
//   * Per-group zero points z ("The 4-bit CPU path", section W4A8: they take
//     the place of the constant 8; W4A16 and grouped W4A8) change only the
//     correction: -z sum xq (int8, exact) or -(1 + z/16) sum x (bf16), from
//     the per-chunk activation sums, with z read for each chunk's group.
//   * Output D[m][n] sits in lane n + 16*(m/4), register m % 4.  The waves'
//     partial results meet in LDS and are added in wave order (integer sums
//     are exact), so a row's bits depend on neither M nor the other rows.
#include <type_traits>

#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

enum class Fmt { W4A16, W4A8, W8A8 };

template <Fmt F> struct Tr;
// CK: k per chunk; ND: MFMAs per chunk; WIN: k per A window (one lane's
// share of one MFMA); XB: bytes per activation value.
template <> struct Tr<Fmt::W4A16> { static constexpr int CK = 128, ND = 4, WIN = 8, XB = 2; };
template <> struct Tr<Fmt::W4A8> { static constexpr int CK = 128, ND = 2, WIN = 16, XB = 1; };
template <> struct Tr<Fmt::W8A8> { static constexpr int CK = 64, ND = 1, WIN = 16, XB = 1; };

constexpr int kNB = 4;              // most chunks one wave owns
constexpr int kSlabBytes = 40 * 1024;
// The whole LDS of a CU (160 KB on gfx950).  Only grouped W4A8 rows longer
// than about 3000 columns pass 64 KB: their per-chunk group sums all wait in
// LDS for the in-order scale epilogue.
constexpr int kMaxLds = 160 * 1024;

struct Args {
  const void *x;        // [M, K] bf16 bits or int8
  const float *sx;      // [M] activation scales (int8 paths)
  const uint8_t *w;     // [N, Kb] packed int4 or int8
  const void *s;        // W4A16: bf16 [N, K/G]; W4A8: f32 [N] or [N, K/G]; W8A8: f32 [N]
  float *yf;            // [M, N] f32 (optional for W4A16)
  uint16_t *yb;         // [M, N] bf16 (W4A16)
  int M, N, K, Kb;      // Kb: bytes per weight row
  int G, GC;            // group size; chunks per group (0: per channel)
  int nC;               // chunks per row
  int slab;             // chunks of activations staged in LDS at a time
  int Mbmax;            // activation rows per block the LDS was sized for
  uint32_t xmask;       // 0x88888888 for two's-complement storage, else 0
  const uint8_t *zp;    // per-group zero points [N, K/G], or null (the constant 8)
  int mx_off;           // fused quantizer: byte offset of the 16 row maxima in LDS
};

__device__ __forceinline__ uint32_t dw(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// One activation window (WIN values of row m from k0); zero when !ok or past
// K.  Straight-line: the address is clamped and the value selected, so the
// compiler can count outstanding loads exactly.
template <Fmt F, bool XV>
__device__ __forceinline__ uint4 load_window(const Args &a, bool ok, int m, int k0) {
  constexpr int WIN = Tr<F>::WIN, XB = Tr<F>::XB;
  const uint8_t *xb = static_cast<const uint8_t *>(a.x);
  if constexpr (XV) {                            // K % WIN == 0, aligned rows
    const bool in = ok && k0 < a.K;
    const uint4 v = load16(xb + (in ? (static_cast<size_t>(m) * a.K + k0) * XB : 0));
    return in ? v : make_uint4(0u, 0u, 0u, 0u);
  }
  // Unaligned rows or a partial last window: the five aligned dwords around
  // the window's 16 bytes, then a byte shift.  A dword is read only if it
  // starts inside the row (so no read leaves the 4-byte block of a byte of
  // x); bytes past K are zero.
  const uintptr_t base = reinterpret_cast<uintptr_t>(xb);
  const size_t row0 = static_cast<size_t>(ok ? m : 0) * a.K * XB;
  const uintptr_t first = base + row0 + static_cast<size_t>(k0) * XB;
  const uintptr_t row_end = base + row0 + static_cast<size_t>(a.K) * XB;
  const uintptr_t a4 = first & ~uintptr_t(3);
  uint32_t d[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const uintptr_t p = a4 + 4 * j;
    const bool rd = ok && p < row_end;
    d[j] = *reinterpret_cast<const uint32_t *>(rd ? p : (base & ~uintptr_t(3)));
    d[j] = rd ? d[j] : 0u;
  }
  const uint32_t sh = static_cast<uint32_t>(first & 3);
  const int nv = ok ? min(max((a.K - k0) * XB, 0), 16) : 0;   // valid bytes of the window
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = __builtin_amdgcn_alignbyte(d[i + 1], d[i], sh);
    const int nb = nv - 4 * i;
    o[i] = nb >= 4 ? v : (nb <= 0 ? 0u : v & ((1u << (8 * nb)) - 1u));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Reorder a window into the k order of the weight unpack.
template <Fmt F>
__device__ __forceinline__ uint4 permute_window(uint4 v) {
  if constexpr (F == Fmt::W4A16) {
    // (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7)
    return make_uint4(perm_b32(v.z, v.x, 0x05040100u), perm_b32(v.z, v.x, 0x07060302u),
                      perm_b32(v.w, v.y, 0x05040100u), perm_b32(v.w, v.y, 0x07060302u));
  } else if constexpr (F == Fmt::W4A8) {
    // bytes 0..15 -> (0,2,4,6)(1,3,5,7)(8,10,12,14)(9,11,13,15)
    return make_uint4(perm_b32(v.y, v.x, 0x06040200u), perm_b32(v.y, v.x, 0x07050301u),
                      perm_b32(v.w, v.z, 0x06040200u), perm_b32(v.w, v.z, 0x07050301u));
  } else {
    return v;
  }
}

// (a & m) | o in one VALU op; m and o live in VGPRs (a literal cannot be
// a VOP3 operand on this architecture, so the compiler would otherwise emit
// a separate and + or).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// bf16 values 1 + u/16 for the 8 nibbles of one dword, in the order
// (n0,n4)(n1,n5)(n2,n6)(n3,n7): each nibble lands in mantissa bits 3..6
// under the exponent of 1.0.
__device__ __forceinline__ uint4 unpack_w4_bf16(uint32_t w, uint32_t M, uint32_t ONE) {
  return make_uint4(and_or(w << 3, M, ONE), and_or(w >> 1, M, ONE), and_or(w >> 5, M, ONE),
                    and_or(w >> 9, M, ONE));
}

// Stored nibbles as bytes: even columns, then odd columns, of each dword.
__device__ __forceinline__ uint4 unpack_w4_i8(uint32_t w0, uint32_t w1) {
  constexpr uint32_t M = 0x0F0F0F0Fu;
  return make_uint4(w0 & M, (w0 >> 4) & M, w1 & M, (w1 >> 4) & M);
}

__device__ __forceinline__ float window_sum_bf16(uint4 v) {
  const float a0 = bf16_to_f32(v.x & 0xFFFFu), a1 = bf16_to_f32(v.x >> 16);
  const float a2 = bf16_to_f32(v.y & 0xFFFFu), a3 = bf16_to_f32(v.y >> 16);
  const float a4 = bf16_to_f32(v.z & 0xFFFFu), a5 = bf16_to_f32(v.z >> 16);
  const float a6 = bf16_to_f32(v.w & 0xFFFFu), a7 = bf16_to_f32(v.w >> 16);
  return ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
}

__device__ __forceinline__ int window_sum_i8(uint4 v) {
  // sum of 16 signed bytes: dot with 0x01 bytes
  int s = 0;
  s = __builtin_amdgcn_sdot4(static_cast<int>(v.x), 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(static_cast<int>(v.y), 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(static_cast<int>(v.z), 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(static_cast<int>(v.w), 0x01010101, s, false);
  return s;
}

// X (W4A8 only): 0 = int8 activation codes with their scales; 1 = f32 and
// 2 = bf16 activations, quantized here with the Q8 recipe: every workgroup
// finds the maxima of its activation rows (one wave per row), then turns
// the windows it stages into codes with the same IEEE operations as the
// standalone quantizer, so codes and scales agree with it bit for bit.
template <Fmt F, int NR, int NW, bool XV, bool TW, int X = 0>
__global__ __launch_bounds__(NW * 64) void gemv_mfma(Args a) {
  static_assert(X == 0 || (F == Fmt::W4A8 && !XV), "the quantizer is fused into W4A8 only");
  using T = Tr<F>;
  constexpr int NT = NW * 64;
  constexpr int WPC = T::ND * 4;          // windows per chunk (4 lane groups x ND)
  constexpr int RW = XV ? NR : 1;         // activation rows loaded before the weights
  constexpr uint32_t XM = TW ? 0x88888888u : 0u;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int q = lane >> 4, ln = lane & 15;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int Mb = NR == 1 ? 1 : (NR == 2 ? 2 : min(16, a.M - m0));
  const int nrow = n0 + ln;
  const int c_begin = (wv * a.nC) / NW, c_end = ((wv + 1) * a.nC) / NW;
  const bool grouped = (F == Fmt::W4A8) && a.GC > 0;
  const int Gn = (F == Fmt::W4A16 || grouped) ? a.K / a.G : 1;

  // LDS: activation windows [slab chunk][window][row] of 16 B, then the
  // per-chunk activation sums [slab chunk][row], then the reduction area.
  // A-operand rows past Mb (and sums of rows past Mb) are read from a valid
  // row instead: they only reach output rows that are never stored.
  uint4 *As = reinterpret_cast<uint4 *>(smem);
  float *Xf = reinterpret_cast<float *>(smem + static_cast<size_t>(a.slab * WPC * a.Mbmax) * 16);
  int *Xi = reinterpret_cast<int *>(Xf);
  constexpr bool kSS = (F != Fmt::W8A8);   // group scales staged (W4A16 always, W4A8 if grouped)
  const bool use_ss = (F == Fmt::W4A16) || grouped;
  uint32_t *Ss = reinterpret_cast<uint32_t *>(Xf + a.slab * a.Mbmax);   // [16 rows][Gn] scale bits
  int *Ri = reinterpret_cast<int *>(Ss + (use_ss ? 16 * Gn : 0));
  float *Rf = reinterpret_cast<float *>(Ri);
  const int arow = NR == 1 ? 0 : ln % Mb;                  // this lane's A row
  const int a_lane = q * T::ND * Mb + arow;                // window index at chunk 0
  int xrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) xrow[r] = NR == 1 ? 0 : (4 * q + r) % Mb;

  const uint32_t M78 = 0x00780078u, ONE = 0x3F803F80u;
  float t[4] = {0.f, 0.f, 0.f, 0.f};   // W4A16 running sum per register
  i32x4 Di = {0, 0, 0, 0};             // per-channel integer accumulator
  int xs[4] = {0, 0, 0, 0};            // per-channel activation sums
  uint4 wb[kNB];                       // this wave's packed weights, all chunks
  int zz[kNB];                         // zero point of each chunk's group (8 without zero points)

  // ---- activation windows: thread -> (chunk, window) slot, rows in turn ----
  uint4 xw[RW];
  // Fused quantizer (X != 0): the whole activation block fits one slab.
  // Wave wv quantizes rows wv, wv + NW, ...; unit (row rr, slot t) of a lane
  // is the 4 values at k = 4 (lane + 64 t), so a load instruction reads
  // consecutive bytes of a row, a window's 4 quarters sit in one lane quad
  // and the 32 quarters of a chunk in 32 consecutive lanes.  The raw values
  // are loaded first and kept in registers; the row maximum is a wave
  // reduction, then the codes are staged as the codes path stages them.
  constexpr int kFU = X == 1 ? 8 : 16;     // units per lane at most
  uint32_t fr[X != 0 ? kFU : 1][X == 1 ? 4 : 2];
  float *Msc = reinterpret_cast<float *>(smem + a.mx_off);   // row scales, for the epilogue
  const int tpr = (a.nC * 32 + 63) / 64;   // unit slots per lane and row
  typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
  typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(2)));
  // unit i of this lane: row m (Mb or more: none) and first column k
  auto funit = [&](int i, int &m, int &k) {
    const int rr = i / tpr, t = i - rr * tpr;
    m = wv + NW * rr;
    k = 4 * (lane + 64 * t);
    if (k >= a.nC * T::CK) m = 16;
  };
  // Every unit is one load at an address inside its row: a whole unit
  // reads its own 4 values; the row's partial last unit reads the row's
  // last 4, and fpick shifts them down by d, with zeros past K (units
  // entirely past K come out zero too).  Only the wave's own rows are read
  // (a bound uniform over the wave), and the values are picked only after
  // the weight loads are issued, so no lane waits between its loads.
  const int nu = ((Mb - wv + NW - 1) / NW) * tpr;   // units of this wave's rows
  auto fload = [&]() {
#pragma unroll
    for (int i = 0; i < kFU; ++i) {
      if (i < nu) {
        const int k = 4 * (lane + 64 * (i % tpr));
        const int mm = wv + NW * (i / tpr);
        const size_t e = static_cast<size_t>(m0 + mm) * a.K + min(k, a.K - 4);   // K >= 4
        if constexpr (X == 1) {
          const u32x4a v = *reinterpret_cast<const u32x4a *>(static_cast<const float *>(a.x) + e);
          fr[i][0] = v.x; fr[i][1] = v.y; fr[i][2] = v.z; fr[i][3] = v.w;
        } else {
          const u32x2a v = *reinterpret_cast<const u32x2a *>(static_cast<const uint16_t *>(a.x) + e);
          fr[i][0] = v.x; fr[i][1] = v.y;
        }
      }
    }
  };
  auto fpick = [&]() {
#pragma unroll
    for (int i = 0; i < kFU; ++i) {
      if (i < nu) {
        const int k = 4 * (lane + 64 * (i % tpr));
        const uint32_t d = static_cast<uint32_t>(k - min(k, a.K - 4));   // 0 for a whole unit
        if constexpr (X == 1) {
          uint32_t v0 = fr[i][0], v1 = fr[i][1], v2 = fr[i][2], v3 = fr[i][3];
          const bool s2 = (d & 2u) != 0, s1 = (d & 1u) != 0, z = d > 3u;
          v0 = s2 ? v2 : v0; v1 = s2 ? v3 : v1; v2 = s2 ? 0u : v2; v3 = s2 ? 0u : v3;
          v0 = s1 ? v1 : v0; v1 = s1 ? v2 : v1; v2 = s1 ? v3 : v2; v3 = s1 ? 0u : v3;
          fr[i][0] = z ? 0u : v0; fr[i][1] = z ? 0u : v1; fr[i][2] = z ? 0u : v2; fr[i][3] = z ? 0u : v3;
        } else {
          const uint64_t w = (static_cast<uint64_t>(fr[i][1]) << 32) | fr[i][0];
          const uint64_t o = d > 3u ? 0ull : w >> (16u * d);
          fr[i][0] = static_cast<uint32_t>(o); fr[i][1] = static_cast<uint32_t>(o >> 32);
        }
      }
    }
  };
  auto fvals = [&](int i, float (&v)[4]) {
    if constexpr (X == 1) {
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) v[t2] = __uint_as_float(fr[i][t2]);
    } else {
      v[0] = bf16_to_f32(fr[i][0] & 0xFFFFu); v[1] = bf16_to_f32(fr[i][0] >> 16);
      v[2] = bf16_to_f32(fr[i][1] & 0xFFFFu); v[3] = bf16_to_f32(fr[i][1] >> 16);
    }
  };
  auto load_rows = [&](int cs, int slot, int r0) {
    const int cl = slot / WPC, j = slot % WPC;
    const int k0 = (cs + cl) * T::CK + j * T::WIN;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int mm = r0 + r;
      if constexpr (X != 0) {
        xw[r] = make_uint4(0u, 0u, 0u, 0u);   // not reached: the fused block is staged whole
        (void)mm; (void)k0;
      } else if constexpr (XV) {
        const bool in = mm < Mb && k0 < a.K;
        xw[r] = load16(static_cast<const uint8_t *>(a.x) +
                       (in ? (static_cast<size_t>(m0 + mm) * a.K + k0) * T::XB : 0));
      } else {
        xw[r] = load_window<F, XV>(a, mm < Mb, m0 + mm, k0);
      }
    }
  };
  auto store_rows = [&](int cs, int slot, int r0) {
    const int cl = slot / WPC, j = slot % WPC;
    const int k0 = (cs + cl) * T::CK + j * T::WIN;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const int mm = r0 + r;
      const bool in = mm < Mb && k0 < a.K;
      const uint4 v = in ? xw[r] : make_uint4(0u, 0u, 0u, 0u);
      if (mm < Mb) As[(cl * WPC + j) * Mb + mm] = permute_window<F>(v);
      if constexpr (F == Fmt::W4A16) {
        const float sm = dpp_row_sum_f32<WPC>(window_sum_bf16(v));
        if (j == 0 && mm < Mb) Xf[cl * Mb + mm] = sm;
      } else if constexpr (F == Fmt::W4A8) {
        const int sm = dpp_row_sum_i32<WPC>(window_sum_i8(v));
        if (j == 0 && mm < Mb) Xi[cl * Mb + mm] = sm;
      }
    }
  };
  // Slots of a slab: SC * WPC; every WPC consecutive threads share a chunk,
  // so the window sums meet in a DPP row reduction among them.
  auto stage_rest = [&](int cs, int first_rows_done) {
    const int SC = min(a.slab, a.nC - cs);
    for (int slot = tid; slot < SC * WPC; slot += NT) {
      for (int r0 = (slot == tid ? first_rows_done : 0); r0 < Mb; r0 += RW) {
        load_rows(cs, slot, r0);
        store_rows(cs, slot, r0);
      }
    }
    lds_barrier();
  };

  // ---- this wave's chunks inside a staged slab ----
  auto compute_slab = [&](int cs) {
    const int SC = min(a.slab, a.nC - cs);
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const int c = c_begin + i;
      if (c >= c_end || c < cs || c >= cs + SC) continue;   // wave-uniform
      const int cl = c - cs;
      uint4 Av[T::ND];
#pragma unroll
      for (int d = 0; d < T::ND; ++d) Av[d] = As[a_lane + (cl * WPC + d) * Mb];
      if constexpr (F == Fmt::W4A16) {
        f32x4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < 4; ++d) D = mfma_bf16_16x16x32(Av[d], unpack_w4_bf16(dw(wb[i], d) ^ XM, M78, ONE), D);
        const float sc = bf16_to_f32(Ss[ln * Gn + c / a.GC]);
        const float bz = -(16.0f + static_cast<float>(zz[i])) * 0.0625f;   // -(1 + z/16); -1.5 at z = 8
#pragma unroll
        for (int r = 0; r < NR; ++r) t[r] = fmaf(sc, fmaf(bz, Xf[cl * Mb + xrow[r]], D[r]), t[r]);
      } else if constexpr (F == Fmt::W4A8) {
        i32x4 D = grouped ? i32x4{0, 0, 0, 0} : Di;
#pragma unroll
        for (int d = 0; d < 2; ++d)
          D = mfma_i8_16x16x64(Av[d], unpack_w4_i8(dw(wb[i], 2 * d) ^ XM, dw(wb[i], 2 * d + 1) ^ XM), D);
        if (grouped) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const int m = 4 * q + r;
            if (m < Mb) Ri[(c * 16 + m) * 16 + ln] = D[r] - zz[i] * Xi[cl * Mb + m];
          }
        } else {
          Di = D;
#pragma unroll
          for (int r = 0; r < NR; ++r) xs[r] += Xi[cl * Mb + xrow[r]];
        }
      } else {
        Di = mfma_i8_16x16x64(Av[0], wb[i], Di);
      }
    }
  };

  // First slab: this thread's first activation rows, then every weight (and
  // scale) load of this wave, all straight-line, so the staging waits only
  // for the activations.  Weight and scale addresses are clamped to valid
  // memory instead of guarded: a clamped piece never matters (rows past N
  // are not stored, pieces past K meet zero activations, chunks outside the
  // wave's range are skipped), and a guard would serialize the loads.
  const int SC0 = min(a.slab, a.nC);
  const bool has0 = X == 0 && tid < SC0 * WPC;
  if (has0) load_rows(0, tid, 0);
  if constexpr (X != 0) fload();
  // The block's group scales: 16 rows x Gn values, contiguous in memory;
  // one coalesced element per thread (clamped index, stored if in range).
  const int sn = 16 * Gn;
  uint32_t sv = 0;
  // the 16 rows are contiguous: a flat index clamped to the matrix end
  const size_t slast = static_cast<size_t>(a.N) * Gn - 1;
  // (the fused kernel loads these unconditionally, at valid clamped
  // addresses, so that the loads between its activation loads and their
  // first use form one straight line whose completions the compiler counts)
  if (X != 0 || (kSS && use_ss)) {
    const size_t src = min(static_cast<size_t>(n0) * Gn + min(tid, sn - 1), slast);
    if constexpr (F == Fmt::W4A16) sv = static_cast<const uint16_t *>(a.s)[src];
    else sv = static_cast<const uint32_t *>(a.s)[src];
  }
  // epilogue operands of the output this thread may own (int paths)
  const int om = tid >> 4, on = tid & 15;
  float sxm = 0.f, swn = 0.f;
  if constexpr (F != Fmt::W4A16 && X == 0) sxm = a.sx[Q4_MUTANT == 7 ? 0 : min(m0 + om, a.M - 1)];   // mutant s07
  if constexpr (F != Fmt::W4A16) {
    if (X != 0 || !grouped) swn = static_cast<const float *>(a.s)[min(n0 + on, a.N - 1)];
  }
  const size_t wrow = static_cast<size_t>(min(nrow, a.N - 1));
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    const int boff = min((c_begin + i) * 64 + q * 16, a.Kb - 16);
    wb[i] = load16(a.w + wrow * a.Kb + boff);
  }
  auto zload = [&]() {
#pragma unroll
    for (int i = 0; i < kNB; ++i) zz[i] = 8;
    if (F != Fmt::W8A8 && a.zp && (F == Fmt::W4A16 || grouped)) {
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        const int c = min(c_begin + i, a.nC - 1);      // clamped like the weights
        zz[i] = a.zp[wrow * Gn + c / a.GC];
      }
    }
  };
  if constexpr (X == 0) zload();
  if (kSS && use_ss) {
    if (tid < sn) Ss[tid] = sv;
    for (int e = tid + NT; e < sn; e += NT) {
      const size_t src = min(static_cast<size_t>(n0) * Gn + e, slast);
      Ss[e] = (F == Fmt::W4A16) ? static_cast<const uint16_t *>(a.s)[src] : static_cast<const uint32_t *>(a.s)[src];
    }
  }
  if constexpr (X != 0) {
    fpick();
    zload();
    // per row of this wave: the maximum over the lanes (fmaxf leaves NaN
    // out, as the standalone quantizer does), the scale RN(max / 127), then
    // the codes: 4 per lane, reordered across the lane pair into the k order
    // of the weight unpack (the codes path's window permutation) and stored
    // a dword per lane, and the chunk's code sum over its 32 lanes
    uint32_t *Aw = reinterpret_cast<uint32_t *>(As);
    const int rpw = (Mb - wv + NW - 1) / NW;   // rows of this wave
    for (int rr = 0; rr < rpw; ++rr) {
      const int mm = wv + NW * rr;
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < kFU; ++i) {
        int m2, k;
        funit(i, m2, k);
        if (m2 != mm) continue;
        float v[4];
        fvals(i, v);
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
      }
      mx = wave_max_f32(mx);
      mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));   // the same in every lane
      const float sc = mx / 127.0f;
      const float rc = q8_row_rcp(mx, sc);
      if (lane == 0) Msc[mm] = sc;
      // the codes of this row; the division form is chosen once per row
      auto codes = [&](auto fast_c) {
        constexpr bool kFast = decltype(fast_c)::value;
#pragma unroll
        for (int i = 0; i < kFU; ++i) {
          int m2, k;
          funit(i, m2, k);
          if (m2 != mm) continue;   // uniform over each group of 32 lanes
          float v[4];
          fvals(i, v);
          // the code as a float in [-127, 127], biased by 128 into a byte
          // (an exact conversion), then the bias flipped off: two's complement
          uint32_t d = 0u;
#pragma unroll
          for (int t2 = 0; t2 < 4; ++t2) {
            const float c = kFast ? q8_code_rcp_f(v[t2], sc, rc) : q8_code_f(v[t2], sc);
            d = __builtin_amdgcn_cvt_pk_u8_f32(c + 128.0f, t2, d);
          }
          d ^= 0x80808080u;
          // window dwords (d0 d1 d2 d3) -> (d0,d1 even bytes)(d0,d1 odd)(d2,d3 even)(d2,d3 odd)
          const uint32_t pd =
              static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(d), 0xB1, 0xF, 0xF, false));
          const bool odd = (lane & 1) != 0;
          const uint32_t lo = odd ? pd : d, hi = odd ? d : pd;
          const int slot = k / T::WIN, cl = slot / WPC, j = slot % WPC;
          Aw[((cl * WPC + j) * Mb + mm) * 4 + (lane & 3)] = perm_b32(hi, lo, odd ? 0x07050301u : 0x06040200u);
          int sm = __builtin_amdgcn_sdot4(static_cast<int>(d), 0x01010101, 0, false);
          sm = dpp_row_sum_i32<16>(sm);
          const auto sw16 = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(sm), static_cast<unsigned>(sm),
                                                             false, false);
          sm = static_cast<int>(sw16[0]) + static_cast<int>(sw16[1]);   // lanes l and l ^ 16
          if ((lane & 31) == 0) Xi[cl * Mb + mm] = sm;
        }
      };
      if (rc != 0.0f) codes(std::true_type{});
      else codes(std::false_type{});
    }
    lds_barrier();
    sxm = Msc[min(om, Mb - 1)];
  } else {
    if (has0) store_rows(0, tid, 0);
    stage_rest(0, RW);
  }
  compute_slab(0);
  for (int cs = a.slab; cs < a.nC; cs += a.slab) {
    lds_barrier();          // every wave is done with the previous slab
    stage_rest(cs, 0);
    compute_slab(cs);
  }

  // ---- combine the waves in a fixed order, then the epilogue ----
  if constexpr (F == Fmt::W4A16) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int m = 4 * q + r;
      if (m < Mb) Rf[(wv * 16 + m) * 16 + ln] = t[r];
    }
  } else if (!grouped) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int m = 4 * q + r;
      if (m < Mb) Ri[(wv * 16 + m) * 16 + ln] = Di[r] - 8 * xs[r];
    }
  }
  __syncthreads();
  if (tid < 256 && om < Mb && n0 + on < a.N) {
    const size_t o = static_cast<size_t>(m0 + om) * a.N + n0 + on;
    if constexpr (F == Fmt::W4A16) {
      float y = Rf[om * 16 + on];
#pragma unroll
      for (int w = 1; w < NW; ++w) y = y + Rf[(w * 16 + om) * 16 + on];
      y = 16.0f * y;
      if (a.yf) a.yf[o] = y;
      a.yb[o] = f32_to_bf16_rne(y);
    } else {
      if (!grouped) {
        int acc = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += Ri[(w * 16 + om) * 16 + on];
        const float tt = static_cast<float>(acc) * sxm;
        a.yf[o] = tt * swn;
      } else {
        const float *sg = reinterpret_cast<const float *>(Ss) + on * Gn;
        float tt = 0.f;
        for (int g = 0; g < Gn; ++g) {
          int acc = 0;
          for (int c = g * a.GC; c < (g + 1) * a.GC; ++c) acc += Ri[(c * 16 + om) * 16 + on];
          const float p = static_cast<float>(acc) * sg[g];
          tt = (g == 0) ? p : tt + p;
        }
        a.yf[o] = tt * sxm;
      }
    }
  }
}

// Waves per workgroup: enough that each wave owns at most kNB chunks.
int waves_for(int nC) {
  if (nC <= 4 * kNB) return 4;
  if (nC <= 8 * kNB) return 8;
  return 16;
}

template <Fmt F>
bool plan(Args &a, int64_t M, int64_t N, int64_t K, int64_t G, size_t *lds, int *nw, bool fused = false) {
  using T = Tr<F>;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(F == Fmt::W8A8 ? K : (K + 1) / 2);
  a.G = static_cast<int>(G);
  a.GC = G > 0 ? static_cast<int>(G / T::CK) : 0;
  a.nC = static_cast<int>((K + T::CK - 1) / T::CK);
  a.Mbmax = static_cast<int>(M < 16 ? M : 16);
  *nw = waves_for(a.nC);
  if (a.nC > 16 * kNB) return false;                       // more chunks than 16 waves hold
  const size_t win_bytes = static_cast<size_t>(T::ND) * 4 * a.Mbmax * 16 + a.Mbmax * 4;  // per chunk
  int slab = static_cast<int>(kSlabBytes / win_bytes);
  if (slab < 1) slab = 1;
  if (slab > a.nC) slab = a.nC;
  a.slab = slab;
  const size_t red = static_cast<size_t>(*nw) * 16 * 16 * 4;
  const size_t grp = (F == Fmt::W4A8 && a.GC > 0) ? static_cast<size_t>(a.nC) * 16 * 16 * 4 : 0;
  const size_t sums = static_cast<size_t>(slab) * a.Mbmax * 4;
  const int64_t gn = (F == Fmt::W4A16 || a.GC > 0) ? K / G : 1;
  const size_t scl = (F == Fmt::W4A16 || a.GC > 0) ? static_cast<size_t>(16 * gn) * 4 : 0;
  *lds = static_cast<size_t>(slab) * T::ND * 4 * a.Mbmax * 16 + sums + scl + (red > grp ? red : grp);
  a.mx_off = static_cast<int>(*lds);
  if (fused) *lds += 16 * 4;   // the row maxima
  return *lds <= kMaxLds;
}

// More than 64 KB of dynamic LDS must be allowed per kernel, once.
template <Fmt F, int NR, int NW, bool XV, bool TW, int X>
bool allow_lds() {
  static const bool ok = hipFuncSetAttribute(reinterpret_cast<const void *>(gemv_mfma<F, NR, NW, XV, TW, X>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             kMaxLds) == hipSuccess;
  return ok;
}

template <Fmt F, int NW, bool XV, bool TW, int X>
hipError_t launch_nw(const Args &a, size_t lds, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.N + 15) / 16), static_cast<unsigned>((a.M + 15) / 16));
  const bool big = lds > 64 * 1024;
  if (a.Mbmax == 1) {
    if (big && !allow_lds<F, 1, NW, XV, TW, X>()) return hipErrorInvalidValue;
    gemv_mfma<F, 1, NW, XV, TW, X><<<grid, NW * 64, lds, st>>>(a);
  } else if (a.Mbmax == 2) {
    if (big && !allow_lds<F, 2, NW, XV, TW, X>()) return hipErrorInvalidValue;
    gemv_mfma<F, 2, NW, XV, TW, X><<<grid, NW * 64, lds, st>>>(a);
  } else {
    if (big && !allow_lds<F, 4, NW, XV, TW, X>()) return hipErrorInvalidValue;
    gemv_mfma<F, 4, NW, XV, TW, X><<<grid, NW * 64, lds, st>>>(a);
  }
  return hipGetLastError();
}

template <Fmt F, bool XV, bool TW, int X = 0>
hipError_t launch_xv(const Args &a, int nw, size_t lds, hipStream_t st) {
  if (nw == 4) return launch_nw<F, 4, XV, TW, X>(a, lds, st);
  if (nw == 8) return launch_nw<F, 8, XV, TW, X>(a, lds, st);
  return launch_nw<F, 16, XV, TW, X>(a, lds, st);
}

template <Fmt F>
hipError_t launch(Args &a, int64_t M, int64_t N, int64_t K, int64_t G, hipStream_t st) {
  size_t lds;
  int nw;
  if (!plan<F>(a, M, N, K, G, &lds, &nw)) return hipErrorInvalidValue;
  const uintptr_t xp = reinterpret_cast<uintptr_t>(a.x);
  const bool xv = (K % Tr<F>::WIN == 0) && (xp % 16 == 0);
  if (F == Fmt::W8A8 || a.xmask == 0)
    return xv ? launch_xv<F, true, false>(a, nw, lds, st) : launch_xv<F, false, false>(a, nw, lds, st);
  return xv ? launch_xv<F, true, true>(a, nw, lds, st) : launch_xv<F, false, true>(a, nw, lds, st);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool gemv_w4a16_ok(const void *x, const void *wq, int64_t K, int64_t G) {
  (void)x;
  if (G <= 0 || G % 128 != 0 || K % G != 0 || !aligned16(wq)) return false;
  Args a{};
  size_t lds;
  int nw;
  return plan<Fmt::W4A16>(a, 16, 16, K, G, &lds, &nw);
}

hipError_t launch_gemv_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                             uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                             hipStream_t st, const uint8_t *zp) {
  Args a{};
  a.x = x; a.w = wq; a.s = s; a.yf = yf; a.yb = yb; a.sx = nullptr; a.zp = zp;
  a.xmask = (enc == kTwos && !zp) ? 0x88888888u : 0u;
  return launch<Fmt::W4A16>(a, M, N, K, G, st);
}

bool gemv_w4a8_ok(const void *wq, int64_t K, int64_t G) {
  if (!aligned16(wq) || ((K + 1) / 2) % 16 != 0) return false;
  if (G != 0 && (G % 128 != 0 || K % G != 0)) return false;
  Args a{};
  size_t lds;
  int nw;
  return plan<Fmt::W4A8>(a, 16, 16, K, G, &lds, &nw);
}

hipError_t launch_gemv_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                            float *y, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                            hipStream_t st, const uint8_t *zp) {
  Args a{};
  a.x = xq; a.sx = sx; a.w = wq; a.s = sw; a.yf = y; a.yb = nullptr; a.zp = G > 0 ? zp : nullptr;
  a.xmask = (enc == kTwos && !a.zp) ? 0x88888888u : 0u;
  return launch<Fmt::W4A8>(a, M, N, K, G, st);
}

// The dynamic W4A8 call quantizes inside the GEMV when a wave's share of
// the raw activation values fits its registers (32 f32 or 64 bf16 values
// per lane: at K = 2048 and four waves, 4 f32 or 8 bf16 rows) and the codes
// one LDS slab.
bool gemv_w4a8_fused_ok(const void *wq, int64_t M, int64_t K, int64_t G, bool x_bf16) {
  if (M < 1 || K < 4 || !gemv_w4a8_ok(wq, K, G)) return false;   // a unit's window is 4 values of its row
  Args a{};
  size_t lds;
  int nw;
  if (!plan<Fmt::W4A8>(a, M, 16, K, G, &lds, &nw, true)) return false;
  const int64_t rows_per_wave = (a.Mbmax + nw - 1) / nw;
  const int64_t slots = (static_cast<int64_t>(a.nC) * 32 + 63) / 64;
  return a.slab >= a.nC && rows_per_wave * slots <= (x_bf16 ? 16 : 8);
}

hipError_t launch_gemv_w4a8_fused(const void *x, bool x_bf16, const uint8_t *wq, const float *sw, float *y,
                                  int64_t M, int64_t N, int64_t K, int64_t G, int enc, hipStream_t st,
                                  const uint8_t *zp) {
  Args a{};
  a.x = x; a.sx = nullptr; a.w = wq; a.s = sw; a.yf = y; a.yb = nullptr; a.zp = G > 0 ? zp : nullptr;
  a.xmask = (enc == kTwos && !a.zp) ? 0x88888888u : 0u;
  size_t lds;
  int nw;
  if (!plan<Fmt::W4A8>(a, M, N, K, G, &lds, &nw, true)) return hipErrorInvalidValue;
  if (x_bf16)
    return a.xmask ? launch_xv<Fmt::W4A8, false, true, 2>(a, nw, lds, st)
                   : launch_xv<Fmt::W4A8, false, false, 2>(a, nw, lds, st);
  return a.xmask ? launch_xv<Fmt::W4A8, false, true, 1>(a, nw, lds, st)
                 : launch_xv<Fmt::W4A8, false, false, 1>(a, nw, lds, st);
}

bool gemv_w8a8_ok(const void *wq, int64_t K) {
  if (!aligned16(wq) || K % 16 != 0) return false;
  Args a{};
  size_t lds;
  int nw;
  return plan<Fmt::W8A8>(a, 16, 16, K, 0, &lds, &nw);
}

hipError_t launch_gemv_w8a8(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw,
                            float *y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  Args a{};
  a.x = xq; a.sx = sx; a.w = reinterpret_cast<const uint8_t *>(wq); a.s = sw; a.yf = y; a.yb = nullptr;
  a.xmask = 0u;
  return launch<Fmt::W8A8>(a, M, N, K, 0, st);
}

}  // namespace q4
