// Device entry points of libq4: argument checks, route choice, launches.
//
// Check order follows the interface of "Fused int4 and int8 dequantize-matmul
// in C" (section 4): invalid arguments first (EINVAL), then the shape rules
// (ESHAPE: K odd, G odd or <= 0, K % G != 0, section 2.2), then M or N == 0
// is a no-op and K == 0 writes y = 0.  Every check runs on the host before
// any HIP call, so a rejected call touches neither the device nor y.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/q4.h"
#include "kernels.hpp"

namespace {

std::atomic<int> g_path{Q4_PATH_AUTO};
thread_local q4_path t_last_path = Q4_PATH_AUTO;

constexpr int64_t kMaxM = 16 * 65535;   // activation rows (grid y of the GEMV kernels)
constexpr int64_t kMaxNK = int64_t(1) << 30;

// Once per device: is it gfx950?  0 = unknown, 1 = yes, 2 = no.
std::atomic<int> g_dev_ok[64];

bool device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int v = g_dev_ok[dev].load(std::memory_order_acquire);
  if (v == 0) {
    hipDeviceProp_t prop;
    v = 2;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
      v = 1;
    g_dev_ok[dev].store(v, std::memory_order_release);
  }
  return v == 1;
}

}  // namespace

bool q4::device_is_gfx950() { return device_ok(); }

namespace {

struct Buf {
  const void *p;
  uint64_t bytes;
};

bool overlap(Buf a, Buf b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Any output overlapping any input, or two outputs overlapping.
bool any_overlap(std::initializer_list<Buf> outs, std::initializer_list<Buf> ins) {
  for (const Buf &o : outs) {
    for (const Buf &i : ins)
      if (overlap(o, i)) return true;
    for (const Buf &o2 : outs)
      if (&o != &o2 && overlap(o, o2)) return true;
  }
  return false;
}

bool bad_dims(int64_t M, int64_t N, int64_t K) { return M < 0 || N < 0 || K < 0; }
bool big_dims(int64_t M, int64_t N, int64_t K) { return M > kMaxM || N > kMaxNK || K > kMaxNK; }
bool bad_enc(int enc) { return enc != Q4_ENC_TWOS && enc != Q4_ENC_EXCESS8; }
bool bad_dt(int xt) { return xt != Q4_DT_F32 && xt != Q4_DT_BF16; }

// The int a C caller passed for an enum parameter.  Comparing the enum
// itself would load a value that may lie outside the enumerators' range,
// which C++ leaves undefined; the bits are read without that load.
template <class E>
int enum_bits(const E &e) {
  static_assert(sizeof(E) == sizeof(int), "enums travel as int");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}
bool grouped_shape_bad(int64_t K, int64_t G) { return K % 2 != 0 || G <= 0 || G % 2 != 0 || K % G != 0; }
uint64_t u(int64_t v) { return static_cast<uint64_t>(v); }

q4_status finish(hipError_t e, q4_path p) {
  if (e != hipSuccess) return Q4_EDEVICE;
  t_last_path = p;
  return Q4_OK;
}

hipStream_t S(void *s) { return static_cast<hipStream_t>(s); }

// ---- route plan ----------------------------------------------------------
//
// Largest batch M that a decode kernel serves before the tiled kernel takes
// over, per measured shape (MI355X, both routes forced, G = 128, hot weights:
// one graph of 20 calls, batch sizes 1..512).  A shape takes the crossing of
// the measured shape nearest to it in (log N, log K); the first of equals
// wins.  Where the weights of one call fit the L2 of an XCD, the decode
// kernels reread them cheaply for every block of 16 rows and keep winning
// up to large M; at N = 13312 and above the tiled kernel wins from its first
// batch (17 rows).  The W4A16 decode kernels serve every M <= 16 on any
// route (the tiled kernels start at 17 rows), so a decode row's bits never
// depend on the batch; integer results are the same on every route.
struct Crossing {
  int32_t N, K;
  int32_t w4a8_grouped, w4a8_channel, w4a16;
};
constexpr Crossing kCrossings[] = {
    // N      K    grouped channel W4A16    time per call at the last decode M,
    //                                      decode / tiled (us), same order
    {2048, 2048, 65, 65, 96},            // 8.7/9.7     6.7/6.7    14.6/16.3
    {5632, 2048, 24, 24, 32},            // 8.8/9.8     6.8/6.8    14.1/16.2
    {13312, 2048, 16, 16, 16},           // tiled from 17 rows (W4A16 at 17: 21.6/20.1)
    {26624, 2048, 16, 16, 16},           // tiled from 17 rows
    {2048, 5632, 32, 32, 32},            // 15.9/22.0   12.4/14.2  21.0/39.6
    {13312, 5632, 16, 16, 16},           // tiled from 17 rows
};

enum class Op { W4A16, W4A8_GROUPED, W4A8_CHANNEL };

int64_t decode_max(Op op, int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return INT64_MAX;
  const Crossing *best = &kCrossings[0];
  double bd = 0.0;
  for (const Crossing &c : kCrossings) {
    const double d = std::fabs(std::log2(static_cast<double>(N) / c.N)) +
                     std::fabs(std::log2(static_cast<double>(K) / c.K));
    if (&c == &kCrossings[0] || d < bd) { bd = d; best = &c; }
  }
  return op == Op::W4A16 ? best->w4a16 : (op == Op::W4A8_GROUPED ? best->w4a8_grouped : best->w4a8_channel);
}

// The forced route, or the measured one: decode up to gemv_max rows, tiled
// above where the shape allows it, the general kernels as the fallback.
q4_path route(bool tiled_ok, bool gemv_ok, int64_t M, int64_t gemv_max) {
  const int forced = g_path.load(std::memory_order_relaxed);
  if (forced == Q4_PATH_GENERIC) return Q4_PATH_GENERIC;
  if (forced == Q4_PATH_TILED) return tiled_ok ? Q4_PATH_TILED : Q4_PATH_GENERIC;
  if (forced == Q4_PATH_GEMV || forced == Q4_PATH_GEMV_MC) return gemv_ok ? Q4_PATH_GEMV : Q4_PATH_GENERIC;
  if (M > gemv_max && tiled_ok) return Q4_PATH_TILED;
  if (gemv_ok) return Q4_PATH_GEMV;
  return Q4_PATH_GENERIC;
}

// Kernel families behind the routes.
enum class Kern { GENERIC, TILED, GEMV_MFMA, GEMV_STREAM, GEMV_MC };

q4_path path_of(Kern k) {
  switch (k) {
    case Kern::TILED: return Q4_PATH_TILED;
    case Kern::GEMV_MFMA:
    case Kern::GEMV_STREAM: return Q4_PATH_GEMV;
    case Kern::GEMV_MC: return Q4_PATH_GEMV_MC;
    default: return Q4_PATH_GENERIC;
  }
}

// W4A16 (zp: zero points given).  The streaming decode kernel is chosen by
// shape, alignment and the route setting, never by M, so a row's bits are
// the same in every batch of up to 16 rows.  The matrix-core decode route
// takes no zero points; such calls take the default decode kernels.
Kern pick_w4a16(const void *x, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G, bool zp) {
  if (!zp && g_path.load(std::memory_order_relaxed) == Q4_PATH_GEMV_MC)
    return q4::gemv_mc_w4a16_ok(x, wq, M, K, G) ? Kern::GEMV_MC : Kern::GENERIC;
  const bool tiled = q4::tiled_w4a16_ok(x, wq, M, N, K, G);
  const bool valu = q4::gemv_stream_w4a16_ok(x, wq, M, K, G);
  const bool mfma = q4::gemv_w4a16_ok(x, wq, K, G);
  const q4_path p = route(tiled, valu || mfma, M, decode_max(Op::W4A16, N, K));
  if (p == Q4_PATH_TILED) return Kern::TILED;
  if (p == Q4_PATH_GEMV) return valu ? Kern::GEMV_STREAM : Kern::GEMV_MFMA;
  return Kern::GENERIC;
}

// One activation row per call is the streaming kernel's on the default route
// (per channel only): from two rows the MFMA GEMV is faster (N = 13312,
// K = 2048: 2 rows 4.1 us against 6.5 us, 8 rows 6.8 against 35).  Forcing
// the decode route gives the streaming kernel every row count it takes
// (tests, A/B), and so does a shape the MFMA GEMV cannot take.
constexpr int64_t kChanStreamMaxM = 1;

// W4A8, per channel (G == 0) or grouped; xq and wq only for alignment.
Kern pick_w4a8(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G) {
  const bool tiled = q4::tiled_w4a8_ok(xq, wq, M, N, K, G);
  const bool mfma = q4::gemv_w4a8_ok(wq, K, G);
  const bool chan = G == 0 && q4::gemv_chan_w4a8_ok(wq, M, K);
  const q4_path p = route(tiled, mfma || chan, M, decode_max(G ? Op::W4A8_GROUPED : Op::W4A8_CHANNEL, N, K));
  if (p == Q4_PATH_TILED) return Kern::TILED;
  if (p != Q4_PATH_GEMV) return Kern::GENERIC;
  const bool stream = chan && (M <= kChanStreamMaxM || !mfma ||
                               g_path.load(std::memory_order_relaxed) == Q4_PATH_GEMV);
  return stream ? Kern::GEMV_STREAM : Kern::GEMV_MFMA;
}

}  // namespace

extern "C" q4_status q4_set_path(q4_path path_arg) {
  const int path = enum_bits(path_arg);
  if (path != Q4_PATH_AUTO && path != Q4_PATH_GENERIC && path != Q4_PATH_GEMV && path != Q4_PATH_TILED &&
      path != Q4_PATH_GEMV_MC)
    return Q4_EINVAL;
  g_path.store(path, std::memory_order_relaxed);
  return Q4_OK;
}

extern "C" q4_path q4_get_path(void) { return static_cast<q4_path>(g_path.load(std::memory_order_relaxed)); }

extern "C" q4_path q4_last_path(void) { return t_last_path; }

extern "C" q4_status q4_route_plan(q4_op op_arg, int64_t M, int64_t N, int64_t K, int64_t G, int32_t cus,
                                   q4_plan *plan) {
  const int op = enum_bits(op_arg);
  if (!plan || bad_dims(M, N, K) || G < 0 || cus < 0) return Q4_EINVAL;
  if (op < Q4_OP_W4A32 || op > Q4_OP_W8A8) return Q4_EINVAL;
  const bool float_grouped = op == Q4_OP_W4A32 || op == Q4_OP_W4A16 || op == Q4_OP_W4A16_ZP;
  if (float_grouped || ((op == Q4_OP_W4A8 || op == Q4_OP_W4A8_ZP) && G > 0)) {
    if (K != 0 && grouped_shape_bad(K, G)) return Q4_ESHAPE;
    if (K == 0 && (G <= 0 || G % 2 != 0)) return Q4_ESHAPE;
  }
  if (op == Q4_OP_W4A8_ZP && G == 0) return Q4_ESHAPE;
  if (big_dims(M, N, K)) return Q4_ESHAPE;
  if ((op == Q4_OP_W4A8 || op == Q4_OP_W4A8_ZP) && K > Q4_W4A8_MAX_K) return Q4_ESHAPE;
  if (op == Q4_OP_W8A8 && K > Q4_W8A8_MAX_K) return Q4_ESHAPE;
  if (cus == 0) {
    if (!device_ok()) return Q4_EDEVICE;
    cus = q4::device_cu_count();
    if (cus <= 0) return Q4_EDEVICE;
  }
  q4_plan p{};
  int64_t dm = INT32_MAX;
  if (float_grouped && op != Q4_OP_W4A32) dm = decode_max(Op::W4A16, N, K);
  if (op == Q4_OP_W4A8 || op == Q4_OP_W4A8_ZP) dm = decode_max(G ? Op::W4A8_GROUPED : Op::W4A8_CHANNEL, N, K);
  p.decode_max = static_cast<int32_t>(dm < INT32_MAX ? dm : INT32_MAX);
  if (M == 0 || N == 0) {
    p.path = Q4_PATH_AUTO;
  } else if (K == 0) {
    p.path = Q4_PATH_GENERIC;
  } else {
    // a nominal 16-byte aligned address for the alignment rules; never read
    const void *al = reinterpret_cast<const void *>(uintptr_t{4096});
    Kern k = Kern::GENERIC;
    if (op == Q4_OP_W4A32) {
      k = route(false, q4::gemv_stream_w4a32_ok(al, al, M, K, G), M, INT64_MAX) == Q4_PATH_GEMV ? Kern::GEMV_STREAM
                                                                                                 : Kern::GENERIC;
    } else if (op == Q4_OP_W4A16 || op == Q4_OP_W4A16_ZP) {
      k = pick_w4a16(al, al, M, N, K, G, op == Q4_OP_W4A16_ZP);
    } else if (op == Q4_OP_W4A8 || op == Q4_OP_W4A8_ZP) {
      k = pick_w4a8(al, al, M, N, K, G);
    } else {
      k = route(false, q4::gemv_w8a8_ok(al, K), M, INT64_MAX) == Q4_PATH_GEMV ? Kern::GEMV_MFMA : Kern::GENERIC;
    }
    p.path = path_of(k);
    if (k == Kern::TILED && (op == Q4_OP_W4A8 || op == Q4_OP_W4A8_ZP)) {
      int full = 0, split = 1;
      int64_t tiles = 0;
      q4::tiled_w4a8_pieces(M, N, cus, &full, &split, &tiles);
      p.whole_tiles = full;
      p.pieces = static_cast<int32_t>((tiles - full) * split);
      p.piece_rows = p.pieces ? 128 / split : 0;
    } else if (k == Kern::TILED) {
      int full = 0;
      int64_t pieces = 0;
      q4::tiled_w4a16_pieces(M, N, cus, &full, &pieces);
      p.whole_tiles = full < 0 ? 0 : full;
      p.pieces = static_cast<int32_t>(pieces);
      p.piece_rows = p.pieces ? 64 : 0;
    }
  }
  *plan = p;
  return Q4_OK;
}

extern "C" q4_status q8_quantize_rows(const void *x, q4_dtype xt_arg, int64_t M, int64_t K, int8_t *xq,
                                      float *sx, void *stream) {
  const int xt = enum_bits(xt_arg);
  if (!x || !xq || !sx || M < 0 || K < 0) return Q4_EINVAL;
  if (bad_dt(xt)) return Q4_EINVAL;
  if (M > kMaxNK || K > kMaxNK) return Q4_ESHAPE;
  const uint64_t xb = u(M) * u(K) * (xt == Q4_DT_BF16 ? 2 : 4);
  if (any_overlap({{xq, u(M) * u(K)}, {sx, u(M) * 4}}, {{x, xb}})) return Q4_EINVAL;
  if (M == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  return finish(q4::launch_quantize_rows(x, xt == Q4_DT_BF16, M, K, xq, sx, S(stream)), Q4_PATH_GEMV);
}

extern "C" q4_status q4_linear_w4a32(const float *x, const uint8_t *wq, const uint16_t *scales_f16,
                                     float *y, int64_t M, int64_t N, int64_t K, int64_t G,
                                     q4_enc enc_arg, void *stream) {
  const int enc = enum_bits(enc_arg);
  if (!x || !wq || !scales_f16 || !y || bad_dims(M, N, K) || bad_enc(enc)) return Q4_EINVAL;
  if (grouped_shape_bad(K, G) && K != 0) return Q4_ESHAPE;
  if (K == 0 && (G <= 0 || G % 2 != 0)) return Q4_ESHAPE;
  if (big_dims(M, N, K)) return Q4_ESHAPE;
  const uint64_t Gn = K ? u(K / G) : 0;
  if (any_overlap({{y, u(M) * u(N) * 4}},
                  {{x, u(M) * u(K) * 4}, {wq, u(N) * u(K / 2)}, {scales_f16, u(N) * Gn * 2}}))
    return Q4_EINVAL;
  if (M == 0 || N == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  if (K == 0) return finish(q4::launch_zero(y, u(M) * u(N) * 4, S(stream)), Q4_PATH_GENERIC);
  // one streaming kernel for every batch size (no tiled f32-activation kernel)
  const bool gemv = q4::gemv_stream_w4a32_ok(x, wq, M, K, G);
  const q4_path p = route(false, gemv, M, INT64_MAX);
  if (p == Q4_PATH_GEMV)
    return finish(q4::launch_gemv_stream_w4a32(x, wq, scales_f16, y, M, N, K, G, enc, S(stream)), p);
  return finish(q4::launch_generic_float(x, false, wq, scales_f16, false, y, nullptr, M, N, K, G, enc,
                                         S(stream)),
                p);
}

namespace {

// W4A16 body shared by the symmetric and the zero-point entry points
// (zp null: the stored nibble decodes by enc; else weight = s * (u - z)).
q4_status w4a16_impl(const uint16_t *x_bf16, const uint8_t *wq, const uint16_t *scales_bf16,
                     const uint8_t *zp, uint16_t *y_bf16, float *y_f32, int64_t M, int64_t N, int64_t K,
                     int64_t G, int enc, void *stream) {
  if (grouped_shape_bad(K, G) && K != 0) return Q4_ESHAPE;
  if (K == 0 && (G <= 0 || G % 2 != 0)) return Q4_ESHAPE;
  if (big_dims(M, N, K)) return Q4_ESHAPE;
  const uint64_t Gn = K ? u(K / G) : 0;
  if (any_overlap({{y_bf16, u(M) * u(N) * 2}, {y_f32, y_f32 ? u(M) * u(N) * 4 : 0}},
                  {{x_bf16, u(M) * u(K) * 2}, {wq, u(N) * u(K / 2)}, {scales_bf16, u(N) * Gn * 2},
                   {zp, zp ? u(N) * Gn : 0}}))
    return Q4_EINVAL;
  if (M == 0 || N == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  hipStream_t st = S(stream);
  if (K == 0) {
    hipError_t e = q4::launch_zero(y_bf16, u(M) * u(N) * 2, st);
    if (e == hipSuccess && y_f32) e = q4::launch_zero(y_f32, u(M) * u(N) * 4, st);
    return finish(e, Q4_PATH_GENERIC);
  }
  switch (pick_w4a16(x_bf16, wq, M, N, K, G, zp != nullptr)) {
    case Kern::GEMV_MC:
      return finish(q4::launch_gemv_mc_w4a16(x_bf16, wq, scales_bf16, y_f32, y_bf16, M, N, K, G, enc, st),
                    Q4_PATH_GEMV_MC);
    case Kern::TILED:
      return finish(q4::launch_tiled_w4a16(x_bf16, wq, scales_bf16, y_f32, y_bf16, M, N, K, G, enc, st, zp),
                    Q4_PATH_TILED);
    case Kern::GEMV_STREAM:
      return finish(q4::launch_gemv_stream_w4a16(x_bf16, wq, scales_bf16, y_f32, y_bf16, M, N, K, G, enc, st, zp),
                    Q4_PATH_GEMV);
    case Kern::GEMV_MFMA:
      return finish(q4::launch_gemv_w4a16(x_bf16, wq, scales_bf16, y_f32, y_bf16, M, N, K, G, enc, st, zp),
                    Q4_PATH_GEMV);
    default:
      return finish(q4::launch_generic_float(x_bf16, true, wq, scales_bf16, true, y_f32, y_bf16, M, N, K, G,
                                             enc, st, zp),
                    Q4_PATH_GENERIC);
  }
}

}  // namespace

extern "C" q4_status q4_linear_w4a16(const uint16_t *x_bf16, const uint8_t *wq,
                                     const uint16_t *scales_bf16, uint16_t *y_bf16, float *y_f32,
                                     int64_t M, int64_t N, int64_t K, int64_t G, q4_enc enc_arg,
                                     void *stream) {
  const int enc = enum_bits(enc_arg);
  if (!x_bf16 || !wq || !scales_bf16 || !y_bf16 || bad_dims(M, N, K) || bad_enc(enc)) return Q4_EINVAL;
  return w4a16_impl(x_bf16, wq, scales_bf16, nullptr, y_bf16, y_f32, M, N, K, G, enc, stream);
}

extern "C" q4_status q4_linear_w4a16_zp(const uint16_t *x_bf16, const uint8_t *wq,
                                        const uint16_t *scales_bf16, const uint8_t *zeros, uint16_t *y_bf16,
                                        float *y_f32, int64_t M, int64_t N, int64_t K, int64_t G,
                                        void *stream) {
  if (!x_bf16 || !wq || !scales_bf16 || !zeros || !y_bf16 || bad_dims(M, N, K)) return Q4_EINVAL;
  return w4a16_impl(x_bf16, wq, scales_bf16, zeros, y_bf16, y_f32, M, N, K, G, Q4_ENC_EXCESS8, stream);
}

namespace {

// xq and sx null with codes_in_scratch: the activation codes live in the
// library's own scratch array, which overlaps no caller buffer.
q4_status w4a8_checks(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                      float *y, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                      std::initializer_list<Buf> extra_ins, bool codes_in_scratch = false) {
  if ((!codes_in_scratch && (!xq || !sx)) || !wq || !sw || !y || bad_dims(M, N, K) || bad_enc(enc) || G < 0)
    return Q4_EINVAL;
  if (G > 0 && grouped_shape_bad(K, G) && K != 0) return Q4_ESHAPE;
  if (G > 0 && K == 0 && G % 2 != 0) return Q4_ESHAPE;
  if (big_dims(M, N, K) || K > Q4_W4A8_MAX_K) return Q4_ESHAPE;
  const uint64_t swn = G > 0 ? u(N) * u(K / G) : u(N);
  const Buf outs = {y, u(M) * u(N) * 4};
  const uint64_t xqb = codes_in_scratch ? 0 : u(M) * u(K), sxb = codes_in_scratch ? 0 : u(M) * 4;
  if (any_overlap({outs}, {{xq, xqb}, {sx, sxb}, {wq, u(N) * u((K + 1) / 2)}, {sw, swn * 4}}))
    return Q4_EINVAL;
  for (const Buf &b : extra_ins)
    if (overlap(outs, b)) return Q4_EINVAL;
  return Q4_OK;
}

// zp: per-group zero points (grouped only).
q4_status w4a8_launch(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw, float *y,
                      int64_t M, int64_t N, int64_t K, int64_t G, int enc, hipStream_t st,
                      const uint8_t *zp = nullptr) {
  if (K == 0) return finish(q4::launch_zero(y, u(M) * u(N) * 4, st), Q4_PATH_GENERIC);
  switch (pick_w4a8(xq, wq, M, N, K, G)) {
    case Kern::TILED:
      return finish(q4::launch_tiled_w4a8(xq, sx, wq, sw, y, M, N, K, G, enc, st, zp), Q4_PATH_TILED);
    case Kern::GEMV_STREAM:
      return finish(q4::launch_gemv_chan_w4a8(xq, 0, sx, wq, sw, y, M, N, K, enc, st), Q4_PATH_GEMV);
    case Kern::GEMV_MFMA:
      return finish(q4::launch_gemv_w4a8(xq, sx, wq, sw, y, M, N, K, G, enc, st, zp), Q4_PATH_GEMV);
    default:
      return finish(q4::launch_generic_int(xq, sx, wq, false, sw, y, M, N, K, G, enc, st, zp), Q4_PATH_GENERIC);
  }
}

}  // namespace

extern "C" q4_status q4_linear_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                                    float *y, int64_t M, int64_t N, int64_t K, int64_t G, q4_enc enc_arg,
                                    void *stream) {
  const int enc = enum_bits(enc_arg);
  const q4_status c = w4a8_checks(xq, sx, wq, sw, y, M, N, K, G, enc, {});
  if (c != Q4_OK) return c;
  if (M == 0 || N == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  return w4a8_launch(xq, sx, wq, sw, y, M, N, K, G, enc, S(stream));
}

extern "C" q4_status q4_linear_w4a8_zp(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                                       const uint8_t *zeros, float *y, int64_t M, int64_t N, int64_t K,
                                       int64_t G, void *stream) {
  if (!zeros) return Q4_EINVAL;
  const uint64_t zb = (G > 0 && K > 0 && K % G == 0) ? u(N) * u(K / G) : 0;
  const q4_status c = w4a8_checks(xq, sx, wq, sw, y, M, N, K, G, Q4_ENC_EXCESS8, {{zeros, zb}});
  if (c != Q4_OK) return c;
  if (G == 0) return Q4_ESHAPE;   // zero points belong to groups
  if (M == 0 || N == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  return w4a8_launch(xq, sx, wq, sw, y, M, N, K, G, Q4_ENC_EXCESS8, S(stream), zeros);
}

namespace {
uint64_t round256(uint64_t v) { return (v + 255) & ~uint64_t(255); }
}  // namespace

extern "C" size_t q4_w4a8_dynamic_workspace(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return static_cast<size_t>(round256(u(M) * u(K)) + round256(u(M) * 4));
}

namespace {

// The library's own workspace for q4_linear_w4a8_dynamic_noalloc: one copy per
// device, alive until the process ends.  In host code `scratch` names a host
// stand-in, never the device array: host code uses only the per-device
// address that hipGetSymbolAddress returns.
static_assert(Q4_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of 256");
__device__ __align__(256) uint8_t scratch[Q4_NOALLOC_SCRATCH_BYTES];

std::atomic<void *> g_scratch[64];
std::mutex g_scratch_mu;

// Address of this device's scratch array (looked up once per device, with
// that device current), or null if the lookup failed.
void *scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    p = q;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Dynamic W4A8 body.  ws is the caller's workspace, or null for the
// library's own scratch array (own_ws), looked up only after every check.
q4_status w4a8_dynamic_impl(const void *x, int xt, const uint8_t *wq, const float *sw, float *y,
                            int64_t M, int64_t N, int64_t K, int64_t G, int enc, void *ws, size_t ws_bytes,
                            bool own_ws, void *stream) {
  if (!x || (!own_ws && !ws) || bad_dt(xt)) return Q4_EINVAL;
  if (M < 0 || K < 0) return Q4_EINVAL;
  const size_t need = q4_w4a8_dynamic_workspace(M, K);
  // codes at offset 0 of the workspace, scales at round256(M K)
  const uint64_t sx_off = round256(u(M) * u(K));
  const uint64_t xb = u(M) * u(K) * (xt == Q4_DT_BF16 ? 2 : 4);
  if (!own_ws) {
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return Q4_EINVAL;
    if (ws_bytes < need) return Q4_EINVAL;
    const Buf wsb = {ws, need};
    const uint64_t swn = G > 0 && K > 0 ? u(N) * u(K / G) : u(N);
    if (any_overlap({wsb}, {{x, xb}, {wq, u(N) * u((K + 1) / 2)}, {sw, swn * 4}, {y, u(M) * u(N) * 4}}))
      return Q4_EINVAL;
    const q4_status c = w4a8_checks(static_cast<int8_t *>(ws),
                                    reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + sx_off), wq, sw, y,
                                    M, N, K, G, enc, {{x, xb}});
    if (c != Q4_OK) return c;
  } else {
    const q4_status c = w4a8_checks(nullptr, nullptr, wq, sw, y, M, N, K, G, enc, {{x, xb}}, true);
    if (c != Q4_OK) return c;
    if (need > Q4_NOALLOC_SCRATCH_BYTES) return Q4_ESHAPE;
  }
  if (M == 0 || N == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  if (own_ws) {
    ws = scratch_ptr();
    if (!ws) return Q4_EDEVICE;
  }
  int8_t *xq = static_cast<int8_t *>(ws);
  float *sx = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + sx_off);
  hipStream_t st = S(stream);
  // Decode: the quantizer runs inside the GEMV (same codes and scales, one
  // launch) on the per-channel streaming kernel, and on the MFMA GEMV while
  // the activation matrix is small; the workspace is then left untouched.
  const Kern k = K > 0 ? pick_w4a8(xq, wq, M, N, K, G) : Kern::GENERIC;
  if (G == 0 && k == Kern::GEMV_STREAM)
    return finish(q4::launch_gemv_chan_w4a8(x, xt == Q4_DT_BF16 ? 2 : 1, nullptr, wq, sw, y, M, N, K, enc, st),
                  Q4_PATH_GEMV);
  if (k == Kern::GEMV_MFMA && q4::gemv_w4a8_fused_ok(wq, M, K, G, xt == Q4_DT_BF16))
    return finish(q4::launch_gemv_w4a8_fused(x, xt == Q4_DT_BF16, wq, sw, y, M, N, K, G, enc, st), Q4_PATH_GEMV);
  const hipError_t e = q4::launch_quantize_rows(x, xt == Q4_DT_BF16, M, K, xq, sx, st);
  if (e != hipSuccess) return Q4_EDEVICE;
  return w4a8_launch(xq, sx, wq, sw, y, M, N, K, G, enc, st);
}

}  // namespace

extern "C" q4_status q4_linear_w4a8_dynamic(const void *x, q4_dtype xt, const uint8_t *wq,
                                            const float *sw, float *y, int64_t M, int64_t N, int64_t K,
                                            int64_t G, q4_enc enc, void *ws, size_t ws_bytes,
                                            void *stream) {
  return w4a8_dynamic_impl(x, enum_bits(xt), wq, sw, y, M, N, K, G, enum_bits(enc), ws, ws_bytes, false, stream);
}

extern "C" q4_status q4_linear_w4a8_dynamic_noalloc(const void *x, q4_dtype xt, const uint8_t *wq,
                                                    const float *sw, float *y, int64_t M, int64_t N,
                                                    int64_t K, int64_t G, q4_enc enc, void *stream) {
  return w4a8_dynamic_impl(x, enum_bits(xt), wq, sw, y, M, N, K, G, enum_bits(enc), nullptr, 0, true, stream);
}

extern "C" q4_status q4_linear_w4a8_dynamic_multi(const q4_w4a8_problem *problems, int64_t count,
                                                  q4_dtype xt_arg, int64_t M, void *stream) {
  const int xt = enum_bits(xt_arg);
  if (count < 0 || count > Q4_MULTI_MAX || (count > 0 && !problems)) return Q4_EINVAL;
  if (bad_dt(xt) || M < 0) return Q4_EINVAL;
  const uint64_t xe = xt == Q4_DT_BF16 ? 2 : 4;
  for (int64_t i = 0; i < count; ++i) {
    const q4_w4a8_problem &p = problems[i];
    if (!p.x || !p.wq || !p.sw || !p.y || p.N < 0 || p.K < 0) return Q4_EINVAL;
    if (reinterpret_cast<uintptr_t>(p.wq) % 16 != 0) return Q4_EINVAL;
  }
  // every output against every input and every other output
  for (int64_t i = 0; i < count; ++i) {
    const q4_w4a8_problem &p = problems[i];
    const Buf yi = {p.y, u(M) * u(p.N) * 4};
    for (int64_t j = 0; j < count; ++j) {
      const q4_w4a8_problem &q = problems[j];
      if (overlap(yi, {q.x, u(M) * u(q.K) * xe}) || overlap(yi, {q.wq, u(q.N) * u((q.K + 1) / 2)}) ||
          overlap(yi, {q.sw, u(q.N) * 4}) || (i != j && overlap(yi, {q.y, u(M) * u(q.N) * 4})))
        return Q4_EINVAL;
    }
  }
  if (M > 16) return Q4_ESHAPE;
  int64_t blocks = 0;
  for (int64_t i = 0; i < count; ++i) {
    const q4_w4a8_problem &p = problems[i];
    if (big_dims(M, p.N, p.K) || p.K > Q4_W4A8_MAX_K) return Q4_ESHAPE;
    if (p.K > 0 && !q4::gemv_chan_w4a8_ok(p.wq, M == 0 ? 1 : M, p.K)) return Q4_ESHAPE;
    blocks += p.K > 0 ? q4::gemv_chan_w4a8_multi_tiles(p.N) : 0;
  }
  if (blocks >= (int64_t(1) << 24)) return Q4_ESHAPE;
  if (M == 0 || count == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  hipStream_t st = S(stream);
  q4::ChanProblem list[Q4_MULTI_MAX];
  int n = 0;
  for (int64_t i = 0; i < count; ++i) {
    const q4_w4a8_problem &p = problems[i];
    if (p.N == 0) continue;
    if (p.K == 0) {
      const hipError_t e = q4::launch_zero(p.y, u(M) * u(p.N) * 4, st);
      if (e != hipSuccess) return Q4_EDEVICE;
      continue;
    }
    list[n++] = {p.x, p.wq, p.sw, p.y, p.N, p.K};
  }
  if (n == 0) return finish(hipSuccess, Q4_PATH_GENERIC);
  return finish(q4::launch_gemv_chan_w4a8_multi(list, n, M, xt == Q4_DT_BF16, st), Q4_PATH_GEMV);
}

namespace {

// W8A32 / W8A16 body: one scale per row, float activations.
q4_status w8_float_impl(const void *x, bool x_bf16, const int8_t *wq, const float *sw, float *y_f32,
                        uint16_t *y_bf16, int64_t M, int64_t N, int64_t K, void *stream) {
  if (big_dims(M, N, K)) return Q4_ESHAPE;
  const uint64_t xb = u(M) * u(K) * (x_bf16 ? 2 : 4);
  if (any_overlap({{y_f32, y_f32 ? u(M) * u(N) * 4 : 0}, {y_bf16, y_bf16 ? u(M) * u(N) * 2 : 0}},
                  {{x, xb}, {wq, u(N) * u(K)}, {sw, u(N) * 4}}))
    return Q4_EINVAL;
  if (M == 0 || N == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  hipStream_t st = S(stream);
  if (K == 0) {
    hipError_t e = hipSuccess;
    if (y_bf16) e = q4::launch_zero(y_bf16, u(M) * u(N) * 2, st);
    if (e == hipSuccess && y_f32) e = q4::launch_zero(y_f32, u(M) * u(N) * 4, st);
    return finish(e, Q4_PATH_GENERIC);
  }
  // one streaming kernel for every batch size (no tiled int8-weight kernel)
  const bool gemv = q4::gemv_stream_w8_ok(x, wq, M, K);
  const q4_path p = route(false, gemv, M, INT64_MAX);
  if (p == Q4_PATH_GEMV)
    return finish(q4::launch_gemv_stream_w8(x, x_bf16, wq, sw, y_f32, y_bf16, M, N, K, st), p);
  return finish(q4::launch_generic_w8_float(x, x_bf16, wq, sw, y_f32, y_bf16, M, N, K, st), p);
}

}  // namespace

extern "C" q4_status q8_linear_w8a32(const float *x, const int8_t *wq, const float *sw, float *y,
                                     int64_t M, int64_t N, int64_t K, void *stream) {
  if (!x || !wq || !sw || !y || bad_dims(M, N, K)) return Q4_EINVAL;
  return w8_float_impl(x, false, wq, sw, y, nullptr, M, N, K, stream);
}

extern "C" q4_status q8_linear_w8a16(const uint16_t *x_bf16, const int8_t *wq, const float *sw,
                                     uint16_t *y_bf16, float *y_f32, int64_t M, int64_t N, int64_t K,
                                     void *stream) {
  if (!x_bf16 || !wq || !sw || !y_bf16 || bad_dims(M, N, K)) return Q4_EINVAL;
  return w8_float_impl(x_bf16, true, wq, sw, y_f32, y_bf16, M, N, K, stream);
}

extern "C" q4_status q8_linear_w8a8(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw,
                                    float *y, int64_t M, int64_t N, int64_t K, void *stream) {
  if (!xq || !sx || !wq || !sw || !y || bad_dims(M, N, K)) return Q4_EINVAL;
  if (big_dims(M, N, K) || K > Q4_W8A8_MAX_K) return Q4_ESHAPE;
  if (any_overlap({{y, u(M) * u(N) * 4}},
                  {{xq, u(M) * u(K)}, {sx, u(M) * 4}, {wq, u(N) * u(K)}, {sw, u(N) * 4}}))
    return Q4_EINVAL;
  if (M == 0 || N == 0) return Q4_OK;
  if (!device_ok()) return Q4_EDEVICE;
  hipStream_t st = S(stream);
  if (K == 0) return finish(q4::launch_zero(y, u(M) * u(N) * 4, st), Q4_PATH_GENERIC);
  const bool gemv = q4::gemv_w8a8_ok(wq, K);
  const q4_path p = route(false, gemv, M, INT64_MAX);
  if (p == Q4_PATH_GEMV) return finish(q4::launch_gemv_w8a8(xq, sx, wq, sw, y, M, N, K, st), p);
  return finish(q4::launch_generic_int(xq, sx, wq, true, sw, y, M, N, K, 0, Q4_ENC_EXCESS8, st), p);
}
