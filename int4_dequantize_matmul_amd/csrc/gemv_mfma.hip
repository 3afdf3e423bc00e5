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
//   * One workgroup = 4 waves owns a block of 16 weight rows and 16
//     activation rows.  Each wave owns a contiguous quarter of the K chunks
//     (a chunk is 64 bytes of every row: 128 int4 or 64 int8 columns), so
//     every lane issues its 16-byte weight loads up front and the packed
//     row is read from HBM exactly once.
//   * The MFMA's B operand is the weights: lane (q, j) holds row j of the
//     block and one 16-byte piece of the chunk.  Nibbles are unpacked in
//     registers with shift-and-mask:
//       int8  MFMA: bytes u = w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F,
//       bf16  MFMA: (w << 3 | w >> 1 | w >> 5 | w >> 9) & 0x00780078 | 0x3F80..,
//                   i.e. the exact bf16 value 1 + u/16 for each stored u.
//     Two's-complement input is first XORed with 0x88888888, which turns it
//     into the excess-8 form (u = t ^ 8 for every nibble).
//   * The A operand is the activations, staged once per workgroup into LDS
//     in the k order the unpack produces, together with per-chunk sums of
//     the activations.  The stored bias then cancels exactly:
//       int8:  sum xq (u - 8)      = D - 8 * sum xq
//       bf16:  sum x (u - 8)       = 16 * (D - 1.5 * sum x)   (v = 1 + u/16)
//   * MFMA output D[m][n] sits in lane n + 16*(m/4), register m % 4; the
//     4 waves' partial results meet in LDS and are combined in a fixed
//     order (integer sums are exact; float partials are added wave 0, 1, 2,
//     3), so a row's bits never depend on M or on the other rows.
#include "kernels.hpp"
#include "q4_device.hpp"

namespace q4 {
namespace {

enum class Fmt { W4A16, W4A8, W8A8 };

template <Fmt F> struct Tr;
// CK: k per chunk; ND: MFMAs per chunk; WIN: k per staged window (one
// lane's share of one MFMA); WPC: windows per chunk; XB: bytes per x value.
template <> struct Tr<Fmt::W4A16> { static constexpr int CK = 128, ND = 4, WIN = 8, WPC = 16, XB = 2; };
template <> struct Tr<Fmt::W4A8> { static constexpr int CK = 128, ND = 2, WIN = 16, WPC = 8, XB = 1; };
template <> struct Tr<Fmt::W8A8> { static constexpr int CK = 64, ND = 1, WIN = 16, WPC = 4, XB = 1; };

constexpr int kNW = 4;            // waves per workgroup
constexpr int kNT = kNW * 64;
constexpr int kNB = 4;            // chunks per weight-load batch
constexpr int kWMAX = 2;          // staged windows per thread loaded before the weights
constexpr int kLdsBudget = 48 * 1024;

struct Args {
  const void *x;        // [M, K] bf16 bits or int8
  const float *sx;      // [M] activation scales (int8 paths)
  const uint8_t *w;     // [N, Kb] packed int4 or int8
  const void *s;        // W4A16: bf16 [N, K/G]; W4A8: f32 [N] or [N, K/G]; W8A8: f32 [N]
  float *yf;            // [M, N] f32 (optional for W4A16)
  uint16_t *yb;         // [M, N] bf16 (W4A16)
  int M, N, K, Kb;      // Kb: bytes per weight row
  int G, GC;            // group size; chunks per group (0: one group of all K)
  int nC;               // chunks per row
  int slab;             // chunks staged in LDS at a time (multiple of GC)
  int Mbmax;            // rows per block the LDS was sized for
  uint32_t xmask;       // 0x88888888 for two's-complement storage, else 0
};

template <Fmt F>
__device__ __forceinline__ uint4 load_window(const Args &a, int m, int k0) {
  constexpr int WIN = Tr<F>::WIN, XB = Tr<F>::XB;
  const uint8_t *base = static_cast<const uint8_t *>(a.x) + (static_cast<size_t>(m) * a.K + k0) * XB;
  if (k0 + WIN <= a.K && (reinterpret_cast<uintptr_t>(base) & 15) == 0) return load16(base);
  uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < WIN; ++e) {
    if (k0 + e < a.K) {
      const uint32_t v = (XB == 2) ? reinterpret_cast<const uint16_t *>(base)[e] : base[e];
      d[(e * XB) >> 2] |= v << (8 * ((e * XB) & 3));
    }
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// Reorder one window into the k order of the weight unpack.
template <Fmt F>
__device__ __forceinline__ uint4 permute_window(uint4 v) {
  if constexpr (F == Fmt::W4A16) {
    // (x0,x1)(x2,x3)(x4,x5)(x6,x7) -> (x0,x4)(x1,x5)(x2,x6)(x3,x7)
    return make_uint4((v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                      (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u));
  } else if constexpr (F == Fmt::W4A8) {
    // bytes 0..15 -> (0,2,4,6)(1,3,5,7)(8,10,12,14)(9,11,13,15)
    return make_uint4(perm_b32(v.y, v.x, 0x06040200u), perm_b32(v.y, v.x, 0x07050301u),
                      perm_b32(v.w, v.z, 0x06040200u), perm_b32(v.w, v.z, 0x07050301u));
  } else {
    return v;
  }
}

__device__ __forceinline__ float window_sum_bf16(uint4 v) {
  const float a0 = bf16_to_f32(v.x & 0xFFFFu), a1 = bf16_to_f32(v.x >> 16);
  const float a2 = bf16_to_f32(v.y & 0xFFFFu), a3 = bf16_to_f32(v.y >> 16);
  const float a4 = bf16_to_f32(v.z & 0xFFFFu), a5 = bf16_to_f32(v.z >> 16);
  const float a6 = bf16_to_f32(v.w & 0xFFFFu), a7 = bf16_to_f32(v.w >> 16);
  return ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
}

__device__ __forceinline__ int window_sum_i8(uint4 v) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) s += static_cast<int8_t>((d[i] >> (8 * b)) & 0xFFu);
  return s;
}

__device__ __forceinline__ uint32_t dw(uint4 v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// bf16 pairs (1 + u/16) for the 8 nibbles of one dword, in the order
// (n0,n4)(n1,n5)(n2,n6)(n3,n7).
__device__ __forceinline__ uint4 unpack_w4_bf16(uint32_t w) {
  constexpr uint32_t M = 0x00780078u, ONE = 0x3F803F80u;
  return make_uint4(((w << 3) & M) | ONE, ((w >> 1) & M) | ONE, ((w >> 5) & M) | ONE,
                    ((w >> 9) & M) | ONE);
}

// Stored nibbles as bytes, even columns then odd columns of each dword.
__device__ __forceinline__ uint4 unpack_w4_i8(uint32_t w0, uint32_t w1) {
  constexpr uint32_t M = 0x0F0F0F0Fu;
  return make_uint4(w0 & M, (w0 >> 4) & M, w1 & M, (w1 >> 4) & M);
}

template <Fmt F, int NR>
__global__ __launch_bounds__(kNT) void gemv_mfma(Args a) {
  using T = Tr<F>;
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int q = lane >> 4, ln = lane & 15;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16;
  const int Mb = min(16, a.M - m0);
  const int nrow = n0 + ln;
  const bool nok = nrow < a.N;
  const int c_begin = (wv * a.nC) / kNW, c_end = ((wv + 1) * a.nC) / kNW;
  const bool grouped = a.GC > 0;
  const int Gn = grouped ? a.K / a.G : 1;

  uint4 *A = reinterpret_cast<uint4 *>(smem);
  float *Xf = reinterpret_cast<float *>(smem + static_cast<size_t>(a.slab) * T::ND * 4 * a.Mbmax * 16);
  int *Xi = reinterpret_cast<int *>(Xf);
  float *Rf = Xf + a.slab * a.Mbmax;
  int *Ri = reinterpret_cast<int *>(Rf);

  // epilogue ownership: thread (om, on) finishes output (m0 + om, n0 + on)
  const int om = tid >> 4, on = tid & 15;
  const bool own = om < Mb && n0 + on < a.N;

  float t[4] = {0.f, 0.f, 0.f, 0.f};   // W4A16 partial per register
  int xs[4] = {0, 0, 0, 0};            // W4A8 activation sums per register
  i32x4 Di = {0, 0, 0, 0};             // integer MFMA accumulator
  float tout = 0.f;                    // grouped W4A8 running f32 sum

  if constexpr (F != Fmt::W4A16) {
    if (!grouped)
      for (int i = tid; i < Mb * 16; i += kNT) Ri[i] = 0;
  }

  for (int cs = 0; cs < a.nC; cs += a.slab) {
    const int SC = min(a.slab, a.nC - cs);
    if constexpr (F == Fmt::W4A8) {
      if (grouped)
        for (int i = tid; i < (SC / a.GC) * Mb * 16; i += kNT) Ri[i] = 0;
    }
    // ---- stage activations: issue the first window loads ----
    const int total = SC * Mb * T::WPC;
    uint4 xw[kWMAX];
#pragma unroll
    for (int i = 0; i < kWMAX; ++i) {
      const int idx = tid + i * kNT;
      if (idx < total) {
        const int j = idx % T::WPC, mm = (idx / T::WPC) % Mb, cl = idx / (T::WPC * Mb);
        xw[i] = load_window<F>(a, m0 + mm, (cs + cl) * T::CK + j * T::WIN);
      }
    }
    // ---- issue this wave's first batch of weight (and scale) loads ----
    const int cb = max(c_begin, cs), ce = min(c_end, cs + SC);
    uint4 wb[kNB];
    uint32_t sb[kNB];
    auto issue = [&](int c0) {
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        const int c = c0 + i;
        const int boff = c * 64 + q * 16;
        wb[i] = (c < ce && nok && boff + 16 <= a.Kb)
                    ? load16(a.w + static_cast<size_t>(nrow) * a.Kb + boff)
                    : make_uint4(0u, 0u, 0u, 0u);
        if constexpr (F == Fmt::W4A16)
          sb[i] = (c < ce && nok)
                      ? static_cast<const uint16_t *>(a.s)[static_cast<size_t>(nrow) * Gn + (c * T::CK) / a.G]
                      : 0u;
      }
    };
    if (cb < ce) issue(cb);
    // ---- finish staging: permute, store, chunk sums ----
    auto stage = [&](int idx, uint4 v) {
      const int j = idx % T::WPC, mm = (idx / T::WPC) % Mb, cl = idx / (T::WPC * Mb);
      const int qq = j / T::ND, d = j % T::ND;
      A[((cl * T::ND + d) * 4 + qq) * Mb + mm] = permute_window<F>(v);
      if constexpr (F == Fmt::W4A16) {
        float s = window_sum_bf16(v);
#pragma unroll
        for (int o = T::WPC / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (j == 0) Xf[cl * Mb + mm] = s;
      } else if constexpr (F == Fmt::W4A8) {
        int s = window_sum_i8(v);
#pragma unroll
        for (int o = T::WPC / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (j == 0) Xi[cl * Mb + mm] = s;
      }
    };
#pragma unroll
    for (int i = 0; i < kWMAX; ++i) {
      const int idx = tid + i * kNT;
      if (idx < total) stage(idx, xw[i]);
    }
    for (int idx = tid + kWMAX * kNT; idx < total; idx += kNT) {
      const int j = idx % T::WPC, mm = (idx / T::WPC) % Mb, cl = idx / (T::WPC * Mb);
      stage(idx, load_window<F>(a, m0 + mm, (cs + cl) * T::CK + j * T::WIN));
    }
    lds_barrier();

    // ---- compute this wave's chunks of the slab ----
    for (int c0 = cb; c0 < ce; c0 += kNB) {
      if (c0 != cb) issue(c0);
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        const int c = c0 + i;
        if (c >= ce) break;
        const int cl = c - cs;
        if constexpr (F == Fmt::W4A16) {
          f32x4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint4 B = unpack_w4_bf16(dw(wb[i], d) ^ a.xmask);
            const uint4 Av = (ln < Mb) ? A[((cl * 4 + d) * 4 + q) * Mb + ln] : make_uint4(0u, 0u, 0u, 0u);
            D = mfma_bf16_16x16x32(Av, B, D);
          }
          const float sc = bf16_to_f32(sb[i]);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const int m = 4 * q + r;
            const float X = (m < Mb) ? Xf[cl * Mb + m] : 0.f;
            const float part = fmaf(-1.5f, X, D[r]);
            t[r] = fmaf(sc, part, t[r]);
          }
        } else if constexpr (F == Fmt::W4A8) {
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const uint4 B = unpack_w4_i8(dw(wb[i], 2 * d) ^ a.xmask, dw(wb[i], 2 * d + 1) ^ a.xmask);
            const uint4 Av = (ln < Mb) ? A[((cl * 2 + d) * 4 + q) * Mb + ln] : make_uint4(0u, 0u, 0u, 0u);
            Di = mfma_i8_16x16x64(Av, B, Di);
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const int m = 4 * q + r;
            xs[r] += (m < Mb) ? Xi[cl * Mb + m] : 0;
          }
          if (grouped && ((c + 1) % a.GC == 0 || c + 1 == ce)) {
            const int gl = (c - cs) / a.GC;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
              const int m = 4 * q + r;
              if (m < Mb) atomicAdd(&Ri[(gl * Mb + m) * 16 + ln], Di[r] - 8 * xs[r]);
              Di[r] = 0;
              xs[r] = 0;
            }
          }
        } else {
          const uint4 Av = (ln < Mb) ? A[(cl * 4 + q) * Mb + ln] : make_uint4(0u, 0u, 0u, 0u);
          Di = mfma_i8_16x16x64(Av, wb[i], Di);
        }
      }
    }
    if constexpr (F == Fmt::W4A8) {
      if (grouped) {
        lds_barrier();
        if (own) {
          const int nslab = SC / a.GC;
          for (int gl = 0; gl < nslab; ++gl) {
            const int g = cs / a.GC + gl;
            const float sg = static_cast<const float *>(a.s)[static_cast<size_t>(n0 + on) * Gn + g];
            const float p = static_cast<float>(Ri[(gl * Mb + om) * 16 + on]) * sg;
            tout = (g == 0) ? p : tout + p;
          }
        }
      }
    }
    lds_barrier();
  }

  // ---- combine the waves and store ----
  if constexpr (F == Fmt::W4A16) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int m = 4 * q + r;
      if (m < Mb) Rf[(wv * Mb + m) * 16 + ln] = t[r];
    }
    lds_barrier();
    if (own) {
      float y = Rf[(0 * Mb + om) * 16 + on];
#pragma unroll
      for (int w = 1; w < kNW; ++w) y = y + Rf[(w * Mb + om) * 16 + on];
      y = 16.0f * y;
      const size_t o = static_cast<size_t>(m0 + om) * a.N + n0 + on;
      if (a.yf) a.yf[o] = y;
      a.yb[o] = f32_to_bf16_rne(y);
    }
  } else {
    const bool pc = (F == Fmt::W8A8) || !grouped;
    if (pc) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int m = 4 * q + r;
        if (m < Mb) atomicAdd(&Ri[m * 16 + ln], Di[r] - 8 * xs[r]);
      }
      lds_barrier();
    }
    if (own) {
      const size_t o = static_cast<size_t>(m0 + om) * a.N + n0 + on;
      const float sxm = a.sx[m0 + om];
      if (pc) {
        const float tt = static_cast<float>(Ri[om * 16 + on]) * sxm;
        a.yf[o] = tt * static_cast<const float *>(a.s)[n0 + on];
      } else {
        a.yf[o] = tout * sxm;
      }
    }
  }
}

template <Fmt F>
bool plan(Args &a, int64_t M, int64_t N, int64_t K, int64_t G, size_t *lds) {
  using T = Tr<F>;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.Kb = static_cast<int>(F == Fmt::W8A8 ? K : (K + 1) / 2);
  a.G = static_cast<int>(G);
  a.GC = G > 0 ? static_cast<int>(G / T::CK) : 0;
  a.nC = static_cast<int>((K + T::CK - 1) / T::CK);
  a.Mbmax = static_cast<int>(M < 16 ? M : 16);
  const size_t per_chunk = static_cast<size_t>(T::ND) * 4 * a.Mbmax * 16 + a.Mbmax * 4 +
                           (a.GC > 0 ? (static_cast<size_t>(a.Mbmax) * 16 * 4 + a.GC - 1) / a.GC : 0);
  int slab = static_cast<int>(kLdsBudget / per_chunk);
  if (a.GC > 0) slab = (slab / a.GC) * a.GC;
  if (slab < 1 || (a.GC > 0 && slab < a.GC)) return false;
  if (slab > a.nC) slab = a.nC > 0 ? a.nC : 1;
  if (a.GC > 0) slab = ((slab + a.GC - 1) / a.GC) * a.GC;   // whole groups per slab
  a.slab = slab;
  size_t r;
  if (F == Fmt::W4A16) r = static_cast<size_t>(kNW) * a.Mbmax * 16 * 4;
  else if (a.GC > 0) r = static_cast<size_t>(slab / a.GC) * a.Mbmax * 16 * 4;
  else r = static_cast<size_t>(a.Mbmax) * 16 * 4;
  *lds = static_cast<size_t>(slab) * T::ND * 4 * a.Mbmax * 16 + static_cast<size_t>(slab) * a.Mbmax * 4 + r;
  return *lds <= 64 * 1024;
}

template <Fmt F>
hipError_t launch(Args &a, size_t lds, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.N + 15) / 16), static_cast<unsigned>((a.M + 15) / 16));
  if (a.Mbmax == 1) gemv_mfma<F, 1><<<grid, kNT, lds, st>>>(a);
  else if (a.Mbmax == 2) gemv_mfma<F, 2><<<grid, kNT, lds, st>>>(a);
  else gemv_mfma<F, 4><<<grid, kNT, lds, st>>>(a);
  return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool gemv_w4a16_ok(const void *x, const void *wq, int64_t K, int64_t G) {
  (void)x;
  if (G <= 0 || G % 128 != 0 || K % G != 0 || !aligned16(wq)) return false;
  Args a{};
  size_t lds;
  return plan<Fmt::W4A16>(a, 16, 16, K, G, &lds);
}

hipError_t launch_gemv_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                             uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                             hipStream_t st) {
  Args a{};
  a.x = x; a.w = wq; a.s = s; a.yf = yf; a.yb = yb; a.sx = nullptr;
  a.xmask = enc == kTwos ? 0x88888888u : 0u;
  size_t lds;
  if (!plan<Fmt::W4A16>(a, M, N, K, G, &lds)) return hipErrorInvalidValue;
  return launch<Fmt::W4A16>(a, lds, st);
}

bool gemv_w4a8_ok(const void *wq, int64_t K, int64_t G) {
  if (!aligned16(wq) || ((K + 1) / 2) % 16 != 0) return false;
  if (G != 0 && (G % 128 != 0 || K % G != 0)) return false;
  Args a{};
  size_t lds;
  return plan<Fmt::W4A8>(a, 16, 16, K, G, &lds);
}

hipError_t launch_gemv_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                            float *y, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                            hipStream_t st) {
  Args a{};
  a.x = xq; a.sx = sx; a.w = wq; a.s = sw; a.yf = y; a.yb = nullptr;
  a.xmask = enc == kTwos ? 0x88888888u : 0u;
  size_t lds;
  if (!plan<Fmt::W4A8>(a, M, N, K, G, &lds)) return hipErrorInvalidValue;
  return launch<Fmt::W4A8>(a, lds, st);
}

bool gemv_w8a8_ok(const void *wq, int64_t K) {
  if (!aligned16(wq) || K % 16 != 0) return false;
  Args a{};
  size_t lds;
  return plan<Fmt::W8A8>(a, 16, 16, K, 0, &lds);
}

hipError_t launch_gemv_w8a8(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw,
                            float *y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  Args a{};
  a.x = xq; a.sx = sx; a.w = reinterpret_cast<const uint8_t *>(wq); a.s = sw; a.yf = y; a.yb = nullptr;
  a.xmask = 0u;
  size_t lds;
  if (!plan<Fmt::W8A8>(a, M, N, K, 0, &lds)) return hipErrorInvalidValue;
  return launch<Fmt::W8A8>(a, lds, st);
}

}  // namespace q4
