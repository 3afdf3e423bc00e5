// Host half of libq4: the load-time quantizers and packer, and the status
// strings.  Plain C++ (no HIP), so it also builds with g++ under ASan/UBSan.
//
// Arithmetic is IEEE binary32 with the default rounding mode: the scale is
// the correctly rounded quotient max|row| / qmax and each code is the
// correctly rounded quotient w / scale, rounded half to even by
// std::nearbyint and clamped to [-qmax, qmax]
// (ftts_kernels module int8, quantize_row_q8; module int4, "The quantization
// contract").  The packed layout is two codes per byte, low nibble = even
// column, stored biased by +8, odd K padded with 8 (module int4, "Packing").
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/q4.h"

namespace {

constexpr int64_t kChunk = 4096;  // codes produced per stack buffer (even)

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

// Scale of one row: max|w| / qmax, correctly rounded.  False for non-finite
// input (checked before anything is written).
bool row_scale(const float *w, int64_t K, int qmax, float *scale) {
  float amax = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    if (!std::isfinite(w[k])) return false;
    const float a = std::fabs(w[k]);
    if (a > amax) amax = a;
  }
  volatile float qm = static_cast<float>(qmax);  // keep the divide a divide
  *scale = amax / qm;
  return true;
}

// Codes of w[0..n) for a given scale: clamp(rint(w / scale)), ties to even.
void row_codes(const float *w, int64_t n, float scale, int qmax, int *codes) {
  const float lim = static_cast<float>(qmax);
  for (int64_t i = 0; i < n; ++i) {
    if (scale == 0.0f) { codes[i] = 0; continue; }
    float r = std::nearbyint(w[i] / scale);  // default mode: nearest, ties to even
    if (r > lim) r = lim;
    if (r < -lim) r = -lim;
    codes[i] = static_cast<int>(r);
  }
}

}  // namespace

extern "C" q4_status q4_quantize_row(const float *w, int64_t K, uint8_t *packed, float *scale) {
  if (!w || !packed || !scale || K < 0) return Q4_EINVAL;
  float s;
  if (!row_scale(w, K, 7, &s)) return Q4_EINVAL;
  int codes[kChunk];
  for (int64_t k0 = 0; k0 < K; k0 += kChunk) {
    const int64_t n = (K - k0 < kChunk) ? (K - k0) : kChunk;
    row_codes(w + k0, n, s, 7, codes);
    for (int64_t i = 0; i < n; i += 2) {  // k0 is even: chunks start on a byte
      const unsigned lo = static_cast<unsigned>(codes[i] + 8);
      const unsigned hi = (i + 1 < n) ? static_cast<unsigned>(codes[i + 1] + 8) : 8u;  // odd-K pad
      packed[(k0 + i) / 2] = static_cast<uint8_t>(lo | (hi << 4));
    }
  }
  *scale = s;
  return Q4_OK;
}

extern "C" q4_status q8_quantize_row(const float *x, int64_t K, int8_t *q, float *scale) {
  if (!x || !q || !scale || K < 0) return Q4_EINVAL;
  float s;
  if (!row_scale(x, K, 127, &s)) return Q4_EINVAL;
  int codes[kChunk];
  for (int64_t k0 = 0; k0 < K; k0 += kChunk) {
    const int64_t n = (K - k0 < kChunk) ? (K - k0) : kChunk;
    row_codes(x + k0, n, s, 127, codes);
    for (int64_t i = 0; i < n; ++i) q[k0 + i] = static_cast<int8_t>(codes[i]);
  }
  *scale = s;
  return Q4_OK;
}

extern "C" q4_status q4_pack(const int8_t *codes, int64_t N, int64_t K, q4_enc enc_arg, uint8_t *packed) {
  const int enc = enum_bits(enc_arg);
  if (!codes || !packed || N < 0 || K < 0) return Q4_EINVAL;
  if (enc != Q4_ENC_TWOS && enc != Q4_ENC_EXCESS8) return Q4_EINVAL;
  if (K > 0 && N > INT64_MAX / K) return Q4_EINVAL;
  for (int64_t i = 0; i < N * K; ++i)
    if (codes[i] < -8 || codes[i] > 7) return Q4_EINVAL;
  const int64_t Kb = (K + 1) / 2;
  const unsigned pad = (enc == Q4_ENC_EXCESS8) ? 8u : 0u;
  for (int64_t n = 0; n < N; ++n) {
    const int8_t *row = codes + n * K;
    for (int64_t b = 0; b < Kb; ++b) {
      auto nib = [&](int64_t k) -> unsigned {
        if (k >= K) return pad;
        const int c = row[k];
        return enc == Q4_ENC_EXCESS8 ? static_cast<unsigned>(c + 8) : static_cast<unsigned>(c & 0xF);
      };
      packed[n * Kb + b] = static_cast<uint8_t>(nib(2 * b) | (nib(2 * b + 1) << 4));
    }
  }
  return Q4_OK;
}

extern "C" const char *q4_status_string(q4_status st_arg) {
  switch (enum_bits(st_arg)) {
    case Q4_OK: return "ok";
    case Q4_EINVAL: return "invalid argument (NULL pointer, negative dimension, unknown enum, overlap or workspace)";
    case Q4_ESHAPE: return "shape rule broken (K odd, G odd or <= 0, K % G != 0, or a size beyond the limits)";
    case Q4_EDEVICE: return "device error (not a gfx950 device, or a HIP launch failed)";
    case Q4_EMISMATCH: return "selftest mismatch (a kernel result differed from its closed form)";
  }
  return "unknown status";
}
