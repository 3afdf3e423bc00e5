// Decode GEMV for per-channel W4A8 (M <= 16) on the vector ALUs, with the
// activation quantizer fused in for float input.
//
// What it computes ("ftts_kernels" module int4: the packing, dot_i32_q4 and
// linear_q4; module int8: quantize_row_q8 and linear_q8_dynamic):
//   acc[m,n] = sum_k xq[m,k] q[n,k]            (exact, i32)
//   y[m,n]   = (f32(acc) * sx[m]) * sw[n]      (two f32 roundings, no FMA)
// where q is the signed code of each stored nibble (excess-8: u - 8; two's
// complement: the nibble itself) and, for float input, sx[m] = max|x[m]|/127
// and xq = clamp(rint(x / sx), -127, 127) exactly as the standalone
// quantizer does (q8_code).  Integer path: bit-exact.
//
// How (gfx950):
//   * A wave owns 4 weight rows; lane l covers columns 32 l .. 32 l + 31 of
//     each 2048-wide pass, one 16-byte nontemporal load per row.
//   * Nibbles become signed bytes 16 q without any bias term:
//       t = stored ^ 0x88888888 (excess-8) or stored (two's complement),
//       high nibbles: t & 0xF0F0F0F0, low nibbles: (t << 4) & 0xF0F0F0F0,
//     so v_dot4_i32_i8 against the activation codes of the even and of the
//     odd columns sums 16 sum xq q exactly; each pass's lane sum is shifted
//     right by 4 (exact) before it joins the running sum.
//   * The workgroup first stages every activation code it needs in LDS, in
//     the order the lanes read them: per row, pass and lane, the codes of
//     the even columns and of the odd columns of each 8-column run.  For
//     float input it takes the row maxima, then quantizes while staging.
//     When a thread's share of the rows fits in registers (the usual decode
//     case) the activations are read once, before the weights are
//     requested, so that waiting for them leaves the weights in flight.
//   * The lane sums meet in a fixed-order integer reduction (exact), and lane
//     0 applies the two scales.
//   * Several independent linears can share one launch: the kernel
//     arguments carry up to 64 problem descriptors and the first workgroup
//     of each; a workgroup finds its problem with one ballot over the lanes
//     and then runs the single-problem body unchanged, so each problem's
//     bits are those of its own call.  One launch per set of linears pays
//     the launch and ramp-up cost once instead of once per linear.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

constexpr int kWaves = 4;             // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kPassK = 2048;          // columns per pass (32 per lane)
constexpr int kMaxLds = 64 * 1024;    // staged activation codes per workgroup
// A row holds 256 staging units per pass; they must split evenly over the
// threads, because the staging loops test only the first unit of each
// round of kThreads units against the total.
static_assert(256 % kThreads == 0, "staging units of a row split evenly over the threads");

enum XT : int { kCodes = 0, kF32 = 1, kBF16 = 2 };

struct CArgs {
  const void *x;        // [M, K]: int8 codes, f32 or bf16
  const float *sx;      // [M] activation scales (codes input only)
  const uint8_t *w;     // [N, Kb] packed nibbles, Kb = ceil(K/2), a multiple of 16
  const float *sw;      // [N]
  float *y;             // [M, N]
  int M, N, K, Kb, npass;
};

typedef unsigned u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16_stream(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p)));
}

__device__ __forceinline__ uint32_t dwc(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Eight float activations of row m from column k0, 0 past K.  Straight-line
// (addresses clamped, values selected), so the compiler can count the
// outstanding loads exactly.  vec (uniform): rows 16-byte aligned, K % 8 == 0.
template <int X>
__device__ __forceinline__ void raw8(const CArgs &a, int m, int k0, bool vec, float (&v)[8]) {
  const bool live = k0 < a.K;   // with vec, the whole run is in or out
  if (vec) {
    const int kc = live ? k0 : 0;
    if constexpr (X == kF32) {
      const float *p = static_cast<const float *>(a.x) + static_cast<size_t>(m) * a.K + kc;
      const float4 u0 = *reinterpret_cast<const float4 *>(p), u1 = *reinterpret_cast<const float4 *>(p + 4);
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w; v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    } else {
      const uint4 u = load16(static_cast<const uint16_t *>(a.x) + static_cast<size_t>(m) * a.K + kc);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_to_f32(dwc(u, i) & 0xFFFFu); v[2 * i + 1] = bf16_to_f32(dwc(u, i) >> 16); }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = live ? v[i] : 0.0f;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + i;
      const size_t idx = static_cast<size_t>(m) * a.K + min(k, a.K - 1);
      float t;
      if constexpr (X == kF32) t = static_cast<const float *>(a.x)[idx];
      else t = bf16_to_f32(static_cast<const uint16_t *>(a.x)[idx]);
      v[i] = k < a.K ? t : 0.0f;
    }
  }
}

// Eight int8 codes of row m from column k0 (0 past K), in column order;
// straight-line as raw8.  vec: rows 8-byte aligned, K % 8 == 0.
__device__ __forceinline__ uint2 raw8codes(const CArgs &a, int m, int k0, bool vec) {
  const int8_t *row = static_cast<const int8_t *>(a.x) + static_cast<size_t>(m) * a.K;
  if (vec) {
    const bool live = k0 < a.K;
    const uint2 c = *reinterpret_cast<const uint2 *>(row + (live ? k0 : 0));
    return live ? c : make_uint2(0u, 0u);
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b0 = static_cast<uint8_t>(row[min(k0 + i, a.K - 1)]);
    const uint32_t b1 = static_cast<uint8_t>(row[min(k0 + 4 + i, a.K - 1)]);
    lo |= (k0 + i < a.K ? b0 : 0u) << (8 * i);
    hi |= (k0 + 4 + i < a.K ? b1 : 0u) << (8 * i);
  }
  return make_uint2(lo, hi);
}

// Codes in column order -> the even-column and the odd-column dwords:
// e = [c0, c2, c4, c6], o = [c1, c3, c5, c7].
__device__ __forceinline__ uint2 split_even_odd(uint2 c) {
  return make_uint2(perm_b32(c.y, c.x, 0x06040200u), perm_b32(c.y, c.x, 0x07050301u));
}

// Eight values -> codes, as the even-column and the odd-column dwords.
// fast is the same for a whole wave (one activation row), so this branches.
__device__ __forceinline__ uint2 code8(const float (&v)[8], float s, float r, bool fast) {
  uint32_t e = 0, o = 0;
  if (fast) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e |= static_cast<uint32_t>(static_cast<uint8_t>(q8_code_rcp(v[2 * i], s, r))) << (8 * i);
      o |= static_cast<uint32_t>(static_cast<uint8_t>(q8_code_rcp(v[2 * i + 1], s, r))) << (8 * i);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e |= static_cast<uint32_t>(static_cast<uint8_t>(q8_code(v[2 * i], s))) << (8 * i);
      o |= static_cast<uint32_t>(static_cast<uint8_t>(q8_code(v[2 * i + 1], s))) << (8 * i);
    }
  }
  return make_uint2(e, o);
}

__device__ __forceinline__ float amax8(const float (&v)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// The single-problem body.  A single call gives every workgroup one tile of
// kWaves * R weight rows (tile `block`).  In a multi-problem launch
// (MULTI) a workgroup takes `tiles` consecutive tiles from tile `block`
// on: the activation codes are staged once for all of them,
// and the (tile, pass) units run as one stream, so the next tile's weights
// are in flight while the current one computes.
template <bool TW, int X, int MP, int R, bool MULTI = false>
__device__ __forceinline__ void chan_body(const CArgs a, unsigned block, int tiles = 1) {
  // codes: [MP][npass][2][64] uint4 (plane h holds the even/odd dwords of
  // the lane's runs 2h and 2h + 1), then the row scales of a codes input
  extern __shared__ __align__(16) unsigned char lds[];
  uint4 *xs = reinterpret_cast<uint4 *>(lds);
  float *scl = reinterpret_cast<float *>(lds + static_cast<size_t>(MP) * a.npass * 2048);
  float *red = scl + 32;   // [kWaves][16] partial maxima (after 16 scales and 16 spare words)

  constexpr uint32_t XM = TW ? 0u : 0x88888888u;   // stored -> two's-complement nibbles
  constexpr int kU = 4;                            // 8-column runs per thread held in registers
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // unit u = (tile u / npass, pass u % npass); the wave's first row in a tile
  const int nunits = MULTI ? tiles * a.npass : a.npass;
  auto tile_of = [&](int u) { return MULTI ? u / a.npass : 0; };
  auto row_of = [&](int t) {
    return MULTI ? static_cast<int>(((block + t) * kWaves + wv) * R) : static_cast<int>((block * kWaves + wv) * R);
  };

  auto load_w = [&](int u, uint4 (&w)[R]) {
    const int t = tile_of(u), p = u - t * a.npass;
    const int n0 = row_of(t);
    const int b = min(p * (kPassK / 2) + 16 * lane, a.Kb - 16);   // past K: a live piece, never used
#pragma unroll
    for (int r = 0; r < R; ++r)
      w[r] = load16_stream(a.w + static_cast<size_t>(min(n0 + r, a.N - 1)) * a.Kb + b);
  };
  // run u = (row m, pass p, lane l, run d) covers columns 8 (u % (256 npass)) + 0..7
  const int per_row = a.npass * 256;
  const int units = a.M * per_row;
  const bool vec = X == kCodes ? (a.K % 8 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 7) == 0)
                               : (a.K % 8 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0);

  // Activations first, then the weights: the wait for the activations then
  // leaves the weights in flight (loads complete in order).  Only raw words
  // are loaded here; decoding them waits until the weights are requested.
  const bool inreg = vec && units <= kU * kThreads;   // the usual decode case
  constexpr int kW = X == kF32 ? 2 : 1;               // 16-byte words per run
  uint4 rr[kU][kW];
  if (inreg) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      if (i * kThreads < units) {
        const int u = tid + i * kThreads;
        const int k0 = 8 * (u % per_row);
        const size_t e = static_cast<size_t>(u / per_row) * a.K + (k0 < a.K ? k0 : 0);
        if constexpr (X == kCodes) {
          const uint2 c = *reinterpret_cast<const uint2 *>(static_cast<const int8_t *>(a.x) + e);
          rr[i][0] = make_uint4(c.x, c.y, 0u, 0u);
        } else if constexpr (X == kF32) {
          rr[i][0] = load16(static_cast<const float *>(a.x) + e);
          rr[i][1] = load16(static_cast<const float *>(a.x) + e + 4);
        } else {
          rr[i][0] = load16(static_cast<const uint16_t *>(a.x) + e);
        }
      }
    }
  }
  uint4 wa[R], wb[R];
  load_w(0, wa);
  if (nunits > 1) load_w(1, wb);
  // raw words of run i -> eight values (0 past K)
  auto decode = [&](int i, float (&v)[8]) {
    const bool live = 8 * ((tid + i * kThreads) % per_row) < a.K;
    if constexpr (X == kF32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[j] = __uint_as_float(dwc(rr[i][0], j)); v[4 + j] = __uint_as_float(dwc(rr[i][1], j)); }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_to_f32(dwc(rr[i][0], j) & 0xFFFFu); v[2 * j + 1] = bf16_to_f32(dwc(rr[i][0], j) >> 16); }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = live ? v[j] : 0.0f;
  };

  if constexpr (X != kCodes) {
    // row maxima over the whole row
    float amax[MP];
#pragma unroll
    for (int m = 0; m < MP; ++m) amax[m] = 0.0f;
    auto note = [&](int m, float mx) {
#pragma unroll
      for (int mm = 0; mm < MP; ++mm)
        if (mm == m) amax[mm] = fmaxf(amax[mm], mx);
    };
    if (inreg) {
#pragma unroll
      for (int i = 0; i < kU; ++i)
        if (i * kThreads < units) {
          float v[8];
          decode(i, v);
          note((tid + i * kThreads) / per_row, amax8(v));
        }
    } else {
      for (int u = tid; u < units; u += kThreads) {
        float v[8];
        raw8<X>(a, u / per_row, 8 * (u % per_row), vec, v);
        note(u / per_row, amax8(v));
      }
    }
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      float v = amax[m];
      v = wave_max_f32(v);
      if (lane == 0) red[wv * 16 + m] = v;
    }
    lds_barrier();
  } else {
    if (tid < MP) scl[tid] = a.sx[min(tid, a.M - 1)];
    lds_barrier();
  }

  // Row m's scale and RN(1 / scale) (0 where the row takes the plain
  // division), formed by every thread that needs them from the per-wave
  // maxima: the same IEEE operations everywhere, so the same values, and
  // no barrier between the maxima and the codes.
  auto row_scale = [&](int m, float &sc, float &r) {
    float v = red[m];
    for (int i = 1; i < kWaves; ++i) v = fmaxf(v, red[i * 16 + m]);
    sc = v / 127.0f;
    r = q8_row_rcp(v, sc);
  };
  float sc0 = 0.0f, r0 = 0.0f;   // row 0, the only row at M = 1
  if constexpr (X != kCodes && MP == 1) {
    row_scale(0, sc0, r0);
    // the same in every lane: keep them in scalar registers
    sc0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sc0)));
    r0 = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r0)));
  }
  auto code_row = [&](int m, const float (&v)[8]) {
    float sc = sc0, r = r0;
    if constexpr (MP > 1) row_scale(m, sc, r);
    return code8(v, sc, r, r != 0.0f);
  };

  // stage the codes in the lanes' reading order
  auto stage = [&](int u, uint2 eo) {
    const int m = u / per_row, r = u % per_row;
    const int p = r / 256, l = (r % 256) / 4, d = r % 4;
    *(reinterpret_cast<uint2 *>(xs + ((m * a.npass + p) * 2 + d / 2) * 64 + l) + (d % 2)) = eo;
  };
  if (inreg) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      if (i * kThreads < units) {
        const int u = tid + i * kThreads;
        if constexpr (X == kCodes) {
          const bool live = 8 * (u % per_row) < a.K;
          stage(u, live ? split_even_odd(make_uint2(rr[i][0].x, rr[i][0].y)) : make_uint2(0u, 0u));
        } else {
          float v[8];
          decode(i, v);
          stage(u, code_row(u / per_row, v));
        }
      }
    }
  } else {
    for (int u = tid; u < units; u += kThreads) {
      if constexpr (X == kCodes) {
        stage(u, split_even_odd(raw8codes(a, u / per_row, 8 * (u % per_row), vec)));
      } else {
        float v[8];
        raw8<X>(a, u / per_row, 8 * (u % per_row), vec, v);
        stage(u, code_row(u / per_row, v));
      }
    }
  }
  lds_barrier();

  int acc[MP][R];
#pragma unroll
  for (int m = 0; m < MP; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0;

  // One pass: the 4 rows' nibbles as signed bytes 16 q (once), then for
  // each activation row two LDS reads and 8 dot4 per weight row.
  auto use = [&](int p, const uint4 (&w)[R]) {
    uint32_t lo[R][4], hi[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t t = dwc(w[r], d) ^ XM;
        hi[r][d] = t & 0xF0F0F0F0u;           // 16 q of the odd columns
        lo[r][d] = (t << 4) & 0xF0F0F0F0u;    // 16 q of the even columns
      }
#pragma unroll
    for (int m = 0; m < MP; ++m) {
      const int mm = min(m, a.M - 1);
      const uint4 v0 = xs[((mm * a.npass + p) * 2 + 0) * 64 + lane];
      const uint4 v1 = xs[((mm * a.npass + p) * 2 + 1) * 64 + lane];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int s = 0;
        s = dot4(lo[r][0], v0.x, s);
        s = dot4(hi[r][0], v0.y, s);
        s = dot4(lo[r][1], v0.z, s);
        s = dot4(hi[r][1], v0.w, s);
        s = dot4(lo[r][2], v1.x, s);
        s = dot4(hi[r][2], v1.y, s);
        s = dot4(lo[r][3], v1.z, s);
        s = dot4(hi[r][3], v1.w, s);
        acc[m][r] += s >> 4;   // s = 16 sum xq q exactly
      }
    }
  };

  // A tile's last pass: exact reduction over the lanes, then the two scales
  // on lane 0; the sums restart for the next tile.
  auto finish = [&](int t) {
#pragma unroll
    for (int m = 0; m < MP; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[m][r] = add_xor32_i32(add_xor16_i32(dpp_row_sum_i32<16>(acc[m][r])));
      }
    if constexpr (!MULTI) {
      if (lane != 0) return;
    }
    if (lane == 0) {
      const int n0 = row_of(t);
#pragma unroll
      for (int m = 0; m < MP; ++m) {
        if (m >= a.M) continue;
        float s = sc0, r;
        if constexpr (X == kCodes) s = scl[m];
        else if constexpr (MP > 1) row_scale(m, s, r);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int n = n0 + r;
          if (n >= a.N) continue;
          // (mutant s08: the activation scale forgotten)
          a.y[static_cast<size_t>(m) * a.N + n] = (static_cast<float>(acc[m][r]) * (Q4_MUTANT == 8 ? 1.0f : s)) * a.sw[n];
        }
      }
    }
    if constexpr (MULTI) {
#pragma unroll
      for (int m = 0; m < MP; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r) acc[m][r] = 0;
    }
  };
  auto use_u = [&](int u, const uint4 (&w)[R]) {
    const int t = tile_of(u), p = u - t * a.npass;
    use(p, w);
    if (p == a.npass - 1) finish(t);
  };

  // units in pairs: wa holds even units, wb odd ones, one unit ahead
  if constexpr (MULTI) {
    int u = 0;
    for (; u + 2 < nunits; u += 2) {
      use_u(u, wa);
      load_w(u + 2, wa);
      use_u(u + 1, wb);
      if (u + 3 < nunits) load_w(u + 3, wb);
    }
    use_u(u, wa);
    if (u + 1 < nunits) use_u(u + 1, wb);
  } else {
    int p = 0;
    for (; p + 2 < a.npass; p += 2) {
      use(p, wa);
      load_w(p + 2, wa);
      use(p + 1, wb);
      if (p + 3 < a.npass) load_w(p + 3, wb);
    }
    use(p, wa);
    if (p + 1 < a.npass) use(p + 1, wb);
    finish(0);
  }
}

template <bool TW, int X, int MP, int R>
__global__ __launch_bounds__(kThreads) void gemv_w4a8_chan(CArgs a) {
  chan_body<TW, X, MP, R>(a, blockIdx.x);
}

// Independent per-channel linears in one launch (float activations,
// excess-8 weights, the same M for all).  Problem i owns workgroups
// first[i] .. first[i+1] - 1; first[0] = 0 and every listed problem has at
// least one workgroup.  A workgroup takes `tiles` tiles of 16 rows (fewer
// at the end of a problem).
constexpr int kMaxMulti = 64;
constexpr int kMultiR = 4;                       // weight rows per wave for every problem
constexpr int kMultiTileRows = kWaves * kMultiR;

struct MProb {
  const void *x;
  const uint8_t *w;
  const float *sw;
  float *y;
  int N, K;
};

struct MArgs {
  MProb p[kMaxMulti];
  int first[kMaxMulti];
  int count, M, tiles;
};
static_assert(sizeof(MArgs) <= 3072, "kernel arguments stay well inside the 4 KB kernarg limit");

template <int X, int MP>
__global__ __launch_bounds__(kThreads) void gemv_w4a8_chan_multi(MArgs a) {
  const int block = blockIdx.x;
  const int lane = threadIdx.x & 63;
  // problem = number of problems i >= 1 whose first workgroup is <= block
  const bool past = lane >= 1 && lane < a.count && a.first[lane < kMaxMulti ? lane : 0] <= block;
  const int i = __builtin_amdgcn_readfirstlane(static_cast<int>(__popcll(__ballot(past))));
  CArgs c{};
  c.x = a.p[i].x;
  c.sx = nullptr;
  c.w = a.p[i].w;
  c.sw = a.p[i].sw;
  c.y = a.p[i].y;
  c.M = a.M;
  c.N = a.p[i].N;
  c.K = a.p[i].K;
  c.Kb = (c.K + 1) / 2;
  c.npass = (c.K + kPassK - 1) / kPassK;
  const int b = block - a.first[i];
  const int left = (c.N - b * a.tiles * kMultiTileRows + kMultiTileRows - 1) / kMultiTileRows;
  chan_body<false, X, MP, kMultiR, true>(c, static_cast<unsigned>(b * a.tiles), min(a.tiles, left));
}

size_t lds_for(int64_t M, int64_t K) {
  const int64_t npass = (K + kPassK - 1) / kPassK;
  int mp = 1;
  while (mp < M) mp *= 2;
  return static_cast<size_t>(mp) * npass * 2048 + 2 * 16 * 4 + kWaves * 16 * 4;
}

template <int X, int MP, int R>
hipError_t launch_r(const CArgs &a, bool tw, hipStream_t st) {
  const size_t lds = lds_for(MP, a.K);
  const dim3 grid(static_cast<unsigned>((a.N + kWaves * R - 1) / (kWaves * R)));
  if (tw) gemv_w4a8_chan<true, X, MP, R><<<grid, kThreads, lds, st>>>(a);
  else gemv_w4a8_chan<false, X, MP, R><<<grid, kThreads, lds, st>>>(a);
  return hipGetLastError();
}

// Rows per wave: as many as keep at least ~256 workgroups in the grid.
template <int X, int MP>
hipError_t launch_x(const CArgs &a, bool tw, hipStream_t st) {
  if (a.N >= 4096) return launch_r<X, MP, 4>(a, tw, st);
  if (a.N >= 2048) return launch_r<X, MP, 2>(a, tw, st);
  return launch_r<X, MP, 1>(a, tw, st);
}

template <int X>
hipError_t launch_m(const CArgs &a, bool tw, hipStream_t st) {
  if (a.M == 1) return launch_x<X, 1>(a, tw, st);
  if (a.M == 2) return launch_x<X, 2>(a, tw, st);
  if (a.M <= 4) return launch_x<X, 4>(a, tw, st);
  if (a.M <= 8) return launch_x<X, 8>(a, tw, st);
  return launch_x<X, 16>(a, tw, st);
}

// Tiles per workgroup.  Measured on the microdecoder pass (35 linears,
// 6720 tiles, M = 1): 1 tile 484 us per 15-pass frame, 2 tiles 452, 3 tiles
// 474, 4 tiles 502 (fewer workgroups than the chip holds at once).  Smaller
// launches keep one tile per workgroup so that they still fill the chip.
constexpr int kMultiTiles = 2;
constexpr int64_t kMultiTilesFrom = 4096;

template <int X>
hipError_t launch_multi(const MArgs &a, unsigned blocks, size_t lds, hipStream_t st) {
  const dim3 grid(blocks);
  if (a.M == 1) gemv_w4a8_chan_multi<X, 1><<<grid, kThreads, lds, st>>>(a);
  else if (a.M == 2) gemv_w4a8_chan_multi<X, 2><<<grid, kThreads, lds, st>>>(a);
  else if (a.M <= 4) gemv_w4a8_chan_multi<X, 4><<<grid, kThreads, lds, st>>>(a);
  else if (a.M <= 8) gemv_w4a8_chan_multi<X, 8><<<grid, kThreads, lds, st>>>(a);
  else gemv_w4a8_chan_multi<X, 16><<<grid, kThreads, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace

int64_t gemv_chan_w4a8_multi_max() { return kMaxMulti; }

int64_t gemv_chan_w4a8_multi_tiles(int64_t N) { return (N + kMultiTileRows - 1) / kMultiTileRows; }

hipError_t launch_gemv_chan_w4a8_multi(const ChanProblem *pr, int count, int64_t M, bool x_bf16,
                                       hipStream_t st) {
  MArgs a{};
  a.count = count;
  a.M = static_cast<int>(M);
  int64_t tiles = 0;
  for (int i = 0; i < count; ++i) tiles += gemv_chan_w4a8_multi_tiles(pr[i].N);
  a.tiles = tiles >= kMultiTilesFrom ? kMultiTiles : 1;
  int64_t blocks = 0, kmax = 0;
  for (int i = 0; i < count; ++i) {
    a.p[i].x = pr[i].x;
    a.p[i].w = pr[i].wq;
    a.p[i].sw = pr[i].sw;
    a.p[i].y = pr[i].y;
    a.p[i].N = static_cast<int>(pr[i].N);
    a.p[i].K = static_cast<int>(pr[i].K);
    a.first[i] = static_cast<int>(blocks);
    blocks += (gemv_chan_w4a8_multi_tiles(pr[i].N) + a.tiles - 1) / a.tiles;
    kmax = pr[i].K > kmax ? pr[i].K : kmax;
  }
  const size_t lds = lds_for(M, kmax);
  const unsigned nb = static_cast<unsigned>(blocks);
  return x_bf16 ? launch_multi<kBF16>(a, nb, lds, st) : launch_multi<kF32>(a, nb, lds, st);
}

bool gemv_chan_w4a8_ok(const void *wq, int64_t M, int64_t K) {
  const int64_t Kb = (K + 1) / 2;
  return M >= 1 && M <= 16 && K > 0 && Kb % 16 == 0 && (reinterpret_cast<uintptr_t>(wq) & 15) == 0 &&
         lds_for(M, K) <= static_cast<size_t>(kMaxLds);
}

hipError_t launch_gemv_chan_w4a8(const void *x, int xt, const float *sx, const uint8_t *wq,
                                 const float *sw, float *y, int64_t M, int64_t N, int64_t K, int enc,
                                 hipStream_t st) {
  CArgs a{};
  a.x = x; a.sx = sx; a.w = wq; a.sw = sw; a.y = y;
  a.M = static_cast<int>(M); a.N = static_cast<int>(N); a.K = static_cast<int>(K);
  a.Kb = static_cast<int>((K + 1) / 2);
  a.npass = static_cast<int>((K + kPassK - 1) / kPassK);
  const bool tw = enc == kTwos;
  if (xt == 0) return launch_m<kCodes>(a, tw, st);
  if (xt == 1) return launch_m<kF32>(a, tw, st);
  return launch_m<kBF16>(a, tw, st);
}

}  // namespace q4
