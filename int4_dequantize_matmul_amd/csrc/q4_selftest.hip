// q4_selftest: all-extreme rows through every kernel route on the running
// GPU, each output compared exactly with its closed form.
//
// Following the tier law of "ftts_kernels" module int8 ("Tier law": every
// tier equals the scalar definition exactly, and a selftest runs the
// all-extreme proof rows through the real kernels on the running silicon to
// show that the i32 reduction cannot overflow at the K values in use).
// Here a "tier" is a kernel route: the general kernels, the streaming and
// MFMA decode GEMVs, the tiled prefill GEMM and the fused activation
// quantizer.  Activation codes are +-127 and weight codes +7, -7 and -8
// (int8 weights +127, -127 and -128), so every product has the largest
// magnitude the formats can hold and every dot product is a closed form:
//   per channel  acc = xq q K (the odd-K pad nibble contributes 0),
//                y = (f32(acc) * sx) * sw
//   grouped      acc_g = xq q G, t = f32(acc_0) s, t = t + f32(acc_g) s in
//                increasing g, y = t * sx
// The largest K tried on each route is the largest that route accepts, so
// the closed forms also prove that no route's accumulator overflows.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/q4.h"
#include "kernels.hpp"

namespace {

thread_local char t_report[1024] = "not run";

// Workspace regions (bytes), each 256-byte aligned.
constexpr size_t kX = size_t(4) << 20;     // activations: 32 x 131072 int8, 2 x 2^20 int8
constexpr size_t kW = size_t(8) << 20;     // weights: 16 x 2^19 packed bytes
constexpr size_t kS = size_t(512) << 10;   // weight scales: 16 x 2^13 f32
constexpr size_t kSX = 256;                // activation scales: 32 f32
constexpr size_t kY = size_t(4) << 10;     // outputs: 32 x 16 f32
constexpr size_t kTotal = kX + kW + kS + kSX + kY;

constexpr int kN = 16;                     // weight rows in every case

struct Ws {
  int8_t *x;
  uint8_t *w;
  float *s;
  float *sx;
  float *y;
};

int8_t act_code(int m) { return (m & 1) ? -127 : 127; }
int w4_code(int n) { return n % 3 == 0 ? 7 : (n % 3 == 1 ? -7 : -8); }
int w8_code(int n) { return n % 3 == 0 ? 127 : (n % 3 == 1 ? -127 : -128); }

// The test runs synchronously on `st`: inputs up, one launch, y down.
struct Runner {
  Ws d;
  hipStream_t st;
  int cases = 0;
  q4_status fail = Q4_OK;
  std::string skipped;   // checks whose shape the route does not take

  void skip(const char *what, int64_t K) {
    char b[96];
    std::snprintf(b, sizeof b, "%s%s K=%lld", skipped.empty() ? "" : "; ", what, static_cast<long long>(K));
    skipped += b;
  }

  bool up(void *dst, const void *src, size_t n) {
    return hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, st) == hipSuccess;
  }

  // Run `launch`, read y [M, kN] and compare with want.
  template <class F>
  void check(const char *what, int64_t K, int64_t M, const std::vector<float> &want, F launch) {
    if (fail != Q4_OK) return;
    std::vector<float> got(static_cast<size_t>(M) * kN, std::nanf(""));
    if (!up(d.y, got.data(), got.size() * 4) || launch() != hipSuccess ||
        hipMemcpyAsync(got.data(), d.y, got.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess) {
      std::snprintf(t_report, sizeof t_report, "%s K=%lld M=%lld: HIP error", what, static_cast<long long>(K),
                    static_cast<long long>(M));
      fail = Q4_EDEVICE;
      return;
    }
    ++cases;
    for (size_t i = 0; i < got.size(); ++i) {
      uint32_t a, b;
      std::memcpy(&a, &got[i], 4);
      std::memcpy(&b, &want[i], 4);
      if (a != b) {
        std::snprintf(t_report, sizeof t_report, "%s K=%lld M=%lld: y[%zu][%zu] = %.9g, closed form %.9g", what,
                      static_cast<long long>(K), static_cast<long long>(M), i / kN, i % kN,
                      static_cast<double>(got[i]), static_cast<double>(want[i]));
        fail = Q4_EMISMATCH;
        return;
      }
    }
  }
};

// Packed rows of one repeated excess-8 code per row; an odd K pads nibble 8.
std::vector<uint8_t> pack_rows(int64_t K) {
  const int64_t Kb = (K + 1) / 2;
  std::vector<uint8_t> w(static_cast<size_t>(kN * Kb));
  for (int n = 0; n < kN; ++n) {
    const uint8_t u = static_cast<uint8_t>(w4_code(n) + 8);
    for (int64_t b = 0; b < Kb; ++b) {
      const uint8_t hi = (2 * b + 1 < K) ? u : 8;
      w[static_cast<size_t>(n * Kb + b)] = static_cast<uint8_t>(u | (hi << 4));
    }
  }
  return w;
}

std::vector<int8_t> act_rows(int64_t M, int64_t K) {
  std::vector<int8_t> x(static_cast<size_t>(M * K));
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) x[static_cast<size_t>(m * K + k)] = act_code(static_cast<int>(m));
  return x;
}

// per channel: y = (f32(acc) * sx) * sw, with sx = sw = 1 or the fused sx
std::vector<float> want_channel(int64_t M, int64_t K, float sx, bool w8) {
  std::vector<float> y(static_cast<size_t>(M) * kN);
  for (int64_t m = 0; m < M; ++m)
    for (int n = 0; n < kN; ++n) {
      const int64_t acc = int64_t(act_code(static_cast<int>(m))) * (w8 ? w8_code(n) : w4_code(n)) * K;
      const float v = static_cast<float>(acc) * sx;
      y[static_cast<size_t>(m * kN + n)] = v * 1.0f;
    }
  return y;
}

// grouped: t = f32(acc_0) * 1; t = t + f32(acc_g) * 1; y = t * 1
std::vector<float> want_grouped(int64_t M, int64_t K, int64_t G) {
  std::vector<float> y(static_cast<size_t>(M) * kN);
  for (int64_t m = 0; m < M; ++m)
    for (int n = 0; n < kN; ++n) {
      const float p = static_cast<float>(int64_t(act_code(static_cast<int>(m))) * w4_code(n) * G) * 1.0f;
      float t = p;
      for (int64_t g = 1; g < K / G; ++g) t = t + p;
      y[static_cast<size_t>(m * kN + n)] = t * 1.0f;
    }
  return y;
}

// The largest K <= cap, a multiple of step, that a route's shape test
// accepts (0 if none).  The tests are not monotone in K (group and pass
// counts matter), so this walks down from the cap.
template <class P>
int64_t largest_k(P ok, int64_t cap, int64_t step) {
  for (int64_t K = cap - cap % step; K >= step; K -= step)
    if (ok(K)) return K;
  return 0;
}

}  // namespace

extern "C" size_t q4_selftest_workspace(void) { return kTotal; }

extern "C" const char *q4_selftest_report(void) { return t_report; }

extern "C" q4_status q4_selftest(void *ws, size_t ws_bytes, void *stream) {
  if (!ws || reinterpret_cast<uintptr_t>(ws) % 256 != 0 || ws_bytes < kTotal) return Q4_EINVAL;
  if (!q4::device_is_gfx950()) return Q4_EDEVICE;
  uint8_t *base = static_cast<uint8_t *>(ws);
  Runner r;
  r.d = {reinterpret_cast<int8_t *>(base), base + kX, reinterpret_cast<float *>(base + kX + kW),
         reinterpret_cast<float *>(base + kX + kW + kS), reinterpret_cast<float *>(base + kX + kW + kS + kSX)};
  r.st = static_cast<hipStream_t>(stream);
  const Ws &d = r.d;
  hipStream_t st = r.st;
  std::vector<float> ones(kS / 4, 1.0f);
  if (!r.up(d.s, ones.data(), kS) || !r.up(d.sx, ones.data(), kSX)) return Q4_EDEVICE;

  // ---- W4A8 per channel and grouped, integer activations ----
  // The configs' K, the tiled kernel's largest per-channel K (131072), the
  // API's largest (Q4_W4A8_MAX_K), and the largest K each decode GEMV takes
  // within what the workspace holds (32 rows of 131072 codes).
  struct KM { int64_t K, M; };
  std::vector<KM> kms = {{1023, 32}, {2048, 32}, {5632, 32}, {131072, 32}, {Q4_W4A8_MAX_K, 2}};
  const int64_t kcap = int64_t(kX) / 32;
  for (const int64_t G : {int64_t(0), int64_t(128)}) {
    const int64_t K = largest_k([&](int64_t k) { return q4::gemv_w4a8_ok(d.w, k, G); }, kcap, 128);
    if (K) kms.push_back({K, 32});
  }
  const int64_t kchan = largest_k([&](int64_t k) { return q4::gemv_chan_w4a8_ok(d.w, 2, k); }, kcap, 32);
  if (kchan) kms.push_back({kchan, 32});
  for (const KM km : kms) {
    const int64_t K = km.K, M = km.M;
    const std::vector<int8_t> x = act_rows(M, K);
    const std::vector<uint8_t> w = pack_rows(K);
    if (!r.up(d.x, x.data(), x.size()) || !r.up(d.w, w.data(), w.size())) return Q4_EDEVICE;
    const std::vector<float> yc = want_channel(M, K, 1.0f, false);
    r.check("w4a8 per channel, generic", K, M, yc, [&] {
      return q4::launch_generic_int(d.x, d.sx, d.w, false, d.s, d.y, M, kN, K, 0, q4::kExcess8, st);
    });
    if (!q4::gemv_w4a8_ok(d.w, K, 0)) r.skip("w4a8 per channel, MFMA GEMV", K);
    else
      r.check("w4a8 per channel, MFMA GEMV", K, M, yc, [&] {
        return q4::launch_gemv_w4a8(d.x, d.sx, d.w, d.s, d.y, M, kN, K, 0, q4::kExcess8, st);
      });
    if (!q4::gemv_chan_w4a8_ok(d.w, 2, K)) r.skip("w4a8 per channel, streaming GEMV", K);
    else
      r.check("w4a8 per channel, streaming GEMV", K, 2, want_channel(2, K, 1.0f, false), [&] {
        return q4::launch_gemv_chan_w4a8(d.x, 0, d.sx, d.w, d.s, d.y, 2, kN, K, q4::kExcess8, st);
      });
    if (!q4::tiled_w4a8_ok(d.x, d.w, M, kN, K, 0)) r.skip("w4a8 per channel, tiled", K);
    else
      r.check("w4a8 per channel, tiled", K, M, yc, [&] {
        return q4::launch_tiled_w4a8(d.x, d.sx, d.w, d.s, d.y, M, kN, K, 0, q4::kExcess8, st);
      });
    if (K % 128 == 0) {
      const std::vector<float> yg = want_grouped(M, K, 128);
      r.check("w4a8 grouped, generic", K, M, yg, [&] {
        return q4::launch_generic_int(d.x, d.sx, d.w, false, d.s, d.y, M, kN, K, 128, q4::kExcess8, st);
      });
      if (!q4::gemv_w4a8_ok(d.w, K, 128)) r.skip("w4a8 grouped, MFMA GEMV", K);
      else
        r.check("w4a8 grouped, MFMA GEMV", K, M, yg, [&] {
          return q4::launch_gemv_w4a8(d.x, d.sx, d.w, d.s, d.y, M, kN, K, 128, q4::kExcess8, st);
        });
      if (!q4::tiled_w4a8_ok(d.x, d.w, M, kN, K, 128)) r.skip("w4a8 grouped, tiled", K);
      else
        r.check("w4a8 grouped, tiled", K, M, yg, [&] {
          return q4::launch_tiled_w4a8(d.x, d.sx, d.w, d.s, d.y, M, kN, K, 128, q4::kExcess8, st);
        });
    }
  }

  // ---- the fused activation quantizer: bf16 rows of +-1 give codes +-127 ----
  for (const int64_t K : {int64_t(1023), int64_t(2048), int64_t(5632), kchan}) {
    if (K == 0) continue;
    const int64_t M = 2;
    std::vector<uint16_t> x(static_cast<size_t>(M * K));
    for (int64_t m = 0; m < M; ++m)
      for (int64_t k = 0; k < K; ++k) x[static_cast<size_t>(m * K + k)] = act_code(static_cast<int>(m)) > 0 ? 0x3F80 : 0xBF80;
    const std::vector<uint8_t> w = pack_rows(K);
    if (!r.up(d.x, x.data(), x.size() * 2) || !r.up(d.w, w.data(), w.size())) return Q4_EDEVICE;
    if (!q4::gemv_chan_w4a8_ok(d.w, M, K)) r.skip("w4a8 per channel, fused quantizer", K);
    else
      r.check("w4a8 per channel, fused quantizer", K, M, want_channel(M, K, 1.0f / 127.0f, false), [&] {
        return q4::launch_gemv_chan_w4a8(d.x, 2, nullptr, d.w, d.s, d.y, M, kN, K, q4::kExcess8, st);
      });
  }

  // ---- W8A8 ----
  std::vector<KM> k8 = {{2048, 32}, {Q4_W8A8_MAX_K, 32}};
  const int64_t k8g = largest_k([&](int64_t k) { return q4::gemv_w8a8_ok(d.w, k); }, Q4_W8A8_MAX_K, 16);
  if (k8g) k8.push_back({k8g, 32});
  for (const KM km : k8) {
    const int64_t K = km.K, M = km.M;
    const std::vector<int8_t> x = act_rows(M, K);
    std::vector<int8_t> w(static_cast<size_t>(kN * K));
    for (int n = 0; n < kN; ++n)
      for (int64_t k = 0; k < K; ++k) w[static_cast<size_t>(n * K + k)] = static_cast<int8_t>(w8_code(n));
    if (!r.up(d.x, x.data(), x.size()) || !r.up(d.w, w.data(), w.size())) return Q4_EDEVICE;
    const std::vector<float> yc = want_channel(M, K, 1.0f, true);
    r.check("w8a8, generic", K, M, yc, [&] {
      return q4::launch_generic_int(d.x, d.sx, d.w, true, d.s, d.y, M, kN, K, 0, q4::kExcess8, st);
    });
    if (!q4::gemv_w8a8_ok(d.w, K)) r.skip("w8a8, MFMA GEMV", K);
    else
      r.check("w8a8, MFMA GEMV", K, M, yc, [&] {
        return q4::launch_gemv_w8a8(d.x, d.sx, reinterpret_cast<const int8_t *>(d.w), d.s, d.y, M, kN, K, st);
      });
  }

  if (r.fail == Q4_OK)
    std::snprintf(t_report, sizeof t_report, "%d route checks passed (all-extreme rows, exact closed forms); "
                  "shapes a route does not take: %s", r.cases, r.skipped.empty() ? "none" : r.skipped.c_str());
  return r.fail;
}
