// Decode GEMV for W4A16 on the matrix cores: M <= 16 activation rows, group
// size 128, 256 or 512.
//
// What it computes ("Fused int4 and int8 dequantize-matmul in C", sections
// 2.2-2.4, with bf16 activations and scales):
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]
// accumulated in f32 and written as f32 and / or bf16 (round to nearest
// even).  A float path, judged by tolerance against the exact value.
//
// How (gfx950):
//   * A workgroup owns RT tiles of 16 weight rows.  K is walked in chunks of
//     2048; within a chunk, each tile is shared by four waves, wave q' taking
//     columns 512 q' .. 512 q' + 511 (four 128-wide subgroups), so a chunk
//     keeps 4 RT waves busy and the grid has ~N/4 waves.  Groups (G | 512)
//     never straddle two waves.
//   * Per chunk the workgroup copies the activations (all M rows) and the
//     group scales of its rows into LDS once (one barrier).
//   * Each lane streams 16 bytes of one weight row per subgroup: lane 16q + c
//     reads bytes 16q..16q+15 of the subgroup's 64 bytes of row c, i.e.
//     columns 32q..32q+31.  Dword d of that piece, unpacked to bf16, is the
//     lane's B operand of one v_mfma_f32_16x16x32_bf16 step; the step pairs
//     lane quarter q with columns 32q + 8d .. 32q + 8d + 7, and the A operand
//     (activation row c of the same 8 columns) is read from LDS with the same
//     mapping.  A matrix product does not care how K is ordered, only that A
//     and B agree.
//   * A stored nibble u (two's complement storage turned into excess-8 by
//     u ^ 8) becomes the bf16 1 + u/16 exactly.  After each step a second
//     MFMA with the constant B operand -1.5 adds -1.5 sum x over the same
//     32 columns to the same accumulator, so it holds
//     sum x (1 + u/16) - 1.5 sum x = sum x (u - 8) / 16; at the end of each
//     group the lane adds acc * 16 s to its running sum.  (The two terms
//     cancel in rounded arithmetic, so a row of zero codes gives a tiny
//     residue rather than an exact zero: a float path, judged by tolerance.)
//   * The output D[m][n] of a step sits in lane n + 16 (m / 4), register
//     m % 4.  The four waves of a tile add their sums through LDS in wave
//     order.  Row m of D depends on row m of A only, and the activation sums
//     are formed per row in a fixed order, so a row's bits do not depend on
//     M; rows beyond M read a clamped row and are never stored.
//   * The next chunk's weights are requested before the current chunk is
//     consumed.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kChunk = 2048;            // k per chunk
constexpr int kSub = kChunk / 128;      // 128-wide subgroups per chunk
constexpr int kKS = 4;                  // waves sharing a row tile (one K quarter of a chunk each)
constexpr int kSubW = kSub / kKS;       // subgroups per wave per chunk = 16-byte loads per lane
constexpr int kXRow = kChunk + 8;       // bf16 per LDS activation row: 16 bytes of pad put
                                        // consecutive rows 4 banks apart
constexpr int kScaleSlots = 16;         // groups a chunk can touch (G >= 128)

struct DArgs {
  const uint16_t *x;    // [M, K] bf16 bits
  const uint8_t *w;     // [N, K/2] packed nibbles
  const uint16_t *s;    // [N, K/G] bf16 bits
  float *yf;            // [M, N] or null
  uint16_t *yb;         // [M, N] or null
  int M, N, K, Kb, G, Gn, nsub, nchunk;
};

template <int MP, int RT>
constexpr int lds_bytes() {
  return MP * kXRow * 2                 // activations of the chunk
         + RT * 16 * kScaleSlots * 4    // 16 s per row and group slot
         + RT * kKS * 64 * 16;          // the waves' partial sums
}

typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

// Weights are read once per call: a nontemporal load keeps them from
// displacing the activations and scales in the caches.
__device__ __forceinline__ uint4 load16_stream(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p)));
}

__device__ __forceinline__ uint32_t dwv(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Dword w of packed weights (8 excess-8 nibbles, low nibble = lower column)
// -> 8 bf16 1 + u/16 in column order.  b * 0x8008 puts the low nibble of a
// byte at bits 3..6 and the high one at 19..22; the masks come in registers
// so that the and-or is a single VOP3 instruction.
__device__ __forceinline__ uint4 unpack_dword(uint32_t w, uint32_t mask, uint32_t one) {
  uint4 r;
  r.x = (((w & 0xFFu) * 0x8008u) & mask) | one;
  r.y = ((((w >> 8) & 0xFFu) * 0x8008u) & mask) | one;
  r.z = ((((w >> 16) & 0xFFu) * 0x8008u) & mask) | one;
  r.w = (((w >> 24) * 0x8008u) & mask) | one;
  return r;
}

template <bool TW, int MP, int RT>
__global__ __launch_bounds__(RT * kKS * 64) void decode_w4a16_mc(DArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  constexpr int kThreads = RT * kKS * 64;
  uint16_t *xs = reinterpret_cast<uint16_t *>(lds);                   // [MP][kXRow]
  float *sc = reinterpret_cast<float *>(lds + MP * kXRow * 2);        // [RT*16][kScaleSlots]: 16 s
  float4 *red = reinterpret_cast<float4 *>(sc + RT * 16 * kScaleSlots);   // [RT][kKS][64]

  constexpr uint32_t XM = TW ? 0x88888888u : 0u;   // two's complement storage -> excess-8
  constexpr int kXL = (MP * kChunk / 8 + kThreads - 1) / kThreads;    // 16-byte activation loads per thread
  constexpr int kSL = (RT * 16 * kScaleSlots + kThreads - 1) / kThreads;   // scale loads per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = wv / kKS;     // row tile
  const int kq = wv % kKS;     // K quarter of each chunk
  const int col = lane & 15;
  const int q = lane >> 4;
  const int nb = blockIdx.x * RT * 16;
  const int n0 = nb + rt * 16;
  const uint8_t *wrow = a.w + static_cast<size_t>(min(n0 + col, a.N - 1)) * a.Kb + 16 * q;
  const int arow = min(col, MP - 1);   // A row this lane supplies (rows past M are clamped copies)
  const int R = a.G / 128;             // subgroups per group

  uint32_t mask = 0x00780078u, one = 0x3F803F80u;
  asm("" : "+v"(mask), "+v"(one));

  auto load_w = [&](int c, uint4 (&w)[kSubW]) {
#pragma unroll
    for (int j = 0; j < kSubW; ++j) {
      const int sub = min(c * kSub + kq * kSubW + j, a.nsub - 1);   // past K: a live piece, never used
      w[j] = load16_stream(wrow + static_cast<size_t>(sub) * 64);
    }
  };
  auto load_x = [&](int c, uint4 (&xr)[kXL]) {
#pragma unroll
    for (int i = 0; i < kXL; ++i) {
      const int e = tid + i * kThreads;                 // 16-byte piece e % 256 of row e / 256
      const int k = min(c * kChunk + 8 * (e & 255), a.K - 8);
      xr[i] = load16(a.x + static_cast<size_t>(min(e >> 8, a.M - 1)) * a.K + k);
    }
  };
  auto load_s = [&](int c, uint32_t (&sr)[kSL]) {
    const int g0 = c * kChunk / a.G;
#pragma unroll
    for (int i = 0; i < kSL; ++i) {
      const int e = min(tid + i * kThreads, RT * 16 * kScaleSlots - 1);   // row e / 16, slot e % 16
      const int n = min(nb + e / kScaleSlots, a.N - 1);
      const int g = min(g0 + e % kScaleSlots, a.Gn - 1);
      sr[i] = a.s[static_cast<size_t>(n) * a.Gn + g];
    }
  };
  // Activations and scales into LDS.  The caller has made sure no wave
  // still reads the previous chunk.
  auto fill = [&](const uint4 (&xr)[kXL], const uint32_t (&sr)[kSL]) {
#pragma unroll
    for (int i = 0; i < kXL; ++i) {
      const int e = tid + i * kThreads;
      if (MP * kChunk / 8 % kThreads == 0 || e < MP * kChunk / 8)
        *reinterpret_cast<uint4 *>(xs + (e >> 8) * kXRow + 8 * (e & 255)) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < kSL; ++i) {
      const int e = tid + i * kThreads;
      if (RT * 16 * kScaleSlots % kThreads == 0 || e < RT * 16 * kScaleSlots)
        sc[e] = 16.0f * bf16_to_f32(sr[i]);
    }
    lds_barrier();
  };

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float t[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint4 kNeg15 = make_uint4(0xBFC0BFC0u, 0xBFC0BFC0u, 0xBFC0BFC0u, 0xBFC0BFC0u);   // bf16 -1.5 x 8

  // This wave's four subgroups of chunk c, four MFMA steps each; group
  // epilogues in order.
  auto consume = [&](int c, const uint4 (&w)[kSubW]) {
#pragma unroll
    for (int jj = 0; jj < kSubW; ++jj) {
      const int j = kq * kSubW + jj;   // subgroup within the chunk
      const int sub = c * kSub + j;
      uint4 aq[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        aq[d] = *reinterpret_cast<const uint4 *>(xs + arow * kXRow + 128 * j + 32 * q + 8 * d);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint4 bq = unpack_dword(dwv(w[jj], d) ^ XM, mask, one);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, aq[d]),
                                                      __builtin_bit_cast(bf16x8v, bq), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, aq[d]),
                                                      __builtin_bit_cast(bf16x8v, kNeg15), acc, 0, 0, 0);
      }
      if ((sub + 1) % R == 0 && sub < a.nsub) {
        const int g = sub / R;
        const float s16 = sc[(rt * 16 + col) * kScaleSlots + g - c * kChunk / a.G];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          t[r] = fmaf(acc[r], s16, t[r]);
          acc[r] = 0.0f;
        }
      }
    }
  };

  // Every load below is unconditional within its straight-line stretch, so
  // the waits for a chunk's activations leave later weight loads in flight.
  uint4 wa[kSubW], wb[kSubW];
  uint4 xr[kXL];
  uint32_t sr[kSL];
  load_x(0, xr);
  load_s(0, sr);
  load_w(0, wa);
  if (a.nchunk == 1) {
    __builtin_amdgcn_sched_barrier(0);
    fill(xr, sr);
    consume(0, wa);
  } else {
    // chunk c's weights in wa (even c) or wb (odd c), requested one chunk ahead
    int c = 0;
    for (; c + 2 < a.nchunk; c += 2) {
      load_w(c + 1, wb);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      fill(xr, sr);
      consume(c, wa);
      load_x(c + 1, xr);
      load_s(c + 1, sr);
      load_w(c + 2, wa);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      fill(xr, sr);
      consume(c + 1, wb);
      load_x(c + 2, xr);
      load_s(c + 2, sr);
    }
    if (c + 1 < a.nchunk) {
      load_w(c + 1, wb);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      fill(xr, sr);
      consume(c, wa);
      load_x(c + 1, xr);
      load_s(c + 1, sr);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      fill(xr, sr);
      consume(c + 1, wb);
    } else {
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      fill(xr, sr);
      consume(c, wa);
    }
  }

  // the four K quarters of a tile meet in LDS and are added in wave order;
  // lane 16q + c then holds rows 4q..4q+3 of column c
  red[wv * 64 + lane] = make_float4(t[0], t[1], t[2], t[3]);
  lds_barrier();
  if (kq != 0) return;
  float4 v = red[rt * kKS * 64 + lane];
#pragma unroll
  for (int i = 1; i < kKS; ++i) {
    const float4 u = red[(rt * kKS + i) * 64 + lane];
    v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
  }
  const float o4[4] = {v.x, v.y, v.z, v.w};
  const int n = n0 + col;
  if (n < a.N) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * q + r;
      if (m < a.M) {
        const size_t o = static_cast<size_t>(m) * a.N + n;
        if (a.yf) a.yf[o] = o4[r];
        if (a.yb) a.yb[o] = f32_to_bf16_rne(o4[r]);
      }
    }
  }
}

template <int MP, int RT>
hipError_t launch_mp(const DArgs &a, bool tw, hipStream_t st) {
  constexpr int bytes = lds_bytes<MP, RT>();
  static const bool attrs = [] {
    bool ok = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_w4a16_mc<true, MP, RT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    ok &= hipFuncSetAttribute(reinterpret_cast<const void *>(decode_w4a16_mc<false, MP, RT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
    return ok;
  }();
  if (!attrs) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((a.N + RT * 16 - 1) / (RT * 16)));
  if (tw) decode_w4a16_mc<true, MP, RT><<<grid, RT * kKS * 64, bytes, st>>>(a);
  else decode_w4a16_mc<false, MP, RT><<<grid, RT * kKS * 64, bytes, st>>>(a);
  return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool gemv_mc_w4a16_ok(const void *x, const void *wq, int64_t M, int64_t K, int64_t G) {
  return M >= 1 && M <= 16 && K > 0 && (G == 128 || G == 256 || G == 512) && K % G == 0 &&
         aligned16(x) && aligned16(wq) && K < (int64_t(1) << 30);
}

hipError_t launch_gemv_mc_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                                uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                                hipStream_t st) {
  DArgs a{};
  a.x = x; a.w = wq; a.s = s; a.yf = yf; a.yb = yb;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(K / 2);
  a.G = static_cast<int>(G);
  a.Gn = static_cast<int>(K / G);
  a.nsub = static_cast<int>(K / 128);
  a.nchunk = static_cast<int>((K + kChunk - 1) / kChunk);
  const bool tw = enc == kTwos;
  if (M == 1) return launch_mp<1, 1>(a, tw, st);
  if (M == 2) return launch_mp<2, 1>(a, tw, st);
  if (M <= 4) return launch_mp<4, 1>(a, tw, st);
  if (M <= 8) return launch_mp<8, 1>(a, tw, st);
  return launch_mp<16, 2>(a, tw, st);
}

}  // namespace q4
