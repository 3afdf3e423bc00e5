// Host quantizers and packer of libq4 under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by test_host_sanitizers.py with g++, no
// device code).  Each output buffer is allocated to its exact size, so a
// write past it is reported by ASan; a canary array after it catches stray
// writes through a valid pointer.  Results are checked for the properties
// that need no oracle: codes in range, the pad nibble, exact negation, and
// rejected rows leaving their outputs untouched.
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "q4.h"

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

// A heap buffer of exactly n bytes (ASan red zones around it).
struct Exact {
  uint8_t *p;
  size_t n;
  explicit Exact(size_t n_) : p(static_cast<uint8_t *>(std::malloc(n_ ? n_ : 1))), n(n_) {
    std::memset(p, 0xA5, n ? n : 1);
  }
  ~Exact() { std::free(p); }
};

static void quantize_rows(std::mt19937 &rng) {
  const int64_t Ks[] = {0, 1, 2, 3, 7, 31, 4095, 4096, 4097, 8191, 8192, 8193, 12289};
  std::normal_distribution<float> nd(0.0f, 1.0f);
  for (int64_t K : Ks) {
    for (float mag : {0.02f, 1.0f, 3.0e38f, 1.0e-40f, 0.0f}) {
      std::vector<float> w(K + 1);   // one spare, so that data() is never NULL (NULL is EINVAL)
      for (auto &v : w) v = nd(rng) * mag;
      if (mag > 1e30f)
        for (auto &v : w) v = std::fmax(std::fmin(v, FLT_MAX), -FLT_MAX);
      Exact packed((K + 1) / 2);
      float s = -1.0f;
      CHECK(q4_quantize_row(w.data(), K, packed.p, &s) == Q4_OK);
      CHECK(s >= 0.0f && std::isfinite(s));
      for (int64_t k = 0; k < K; ++k) {
        const unsigned u = (packed.p[k / 2] >> (4 * (k & 1))) & 0xF;
        CHECK(u >= 1 && u <= 15);                  // excess-8 codes -7..7
      }
      if (K % 2) CHECK((packed.p[K / 2] >> 4) == 8);  // the pad nibble
      // negation gives the same scale and negated codes
      std::vector<float> wn(K + 1);
      for (int64_t k = 0; k <= K; ++k) wn[k] = -w[k];
      Exact pn((K + 1) / 2);
      float sn = -1.0f;
      CHECK(q4_quantize_row(wn.data(), K, pn.p, &sn) == Q4_OK);
      CHECK(sn == s);
      for (int64_t k = 0; k < K; ++k) {
        const int q = static_cast<int>((packed.p[k / 2] >> (4 * (k & 1))) & 0xF) - 8;
        const int qn = static_cast<int>((pn.p[k / 2] >> (4 * (k & 1))) & 0xF) - 8;
        CHECK(qn == -q);
      }
      Exact q8(K);
      float s8 = -1.0f;
      CHECK(q8_quantize_row(w.data(), K, reinterpret_cast<int8_t *>(q8.p), &s8) == Q4_OK);
      for (int64_t k = 0; k < K; ++k) {
        const int c = static_cast<int8_t>(q8.p[k]);
        CHECK(c >= -127 && c <= 127);
      }
    }
  }
}

static void rejected_rows() {
  for (float bad : {NAN, INFINITY, -INFINITY}) {
    for (int64_t K : {1, 4096, 4097}) {
      std::vector<float> w(K, 0.5f);
      w[K - 1] = bad;
      Exact packed((K + 1) / 2);
      Exact q8(K);
      float s = 7.0f, s8 = 7.0f;
      CHECK(q4_quantize_row(w.data(), K, packed.p, &s) == Q4_EINVAL);
      CHECK(q8_quantize_row(w.data(), K, reinterpret_cast<int8_t *>(q8.p), &s8) == Q4_EINVAL);
      CHECK(s == 7.0f && s8 == 7.0f);
      for (size_t i = 0; i < packed.n; ++i) CHECK(packed.p[i] == 0xA5);
      for (size_t i = 0; i < q8.n; ++i) CHECK(q8.p[i] == 0xA5);
    }
  }
  float s = 0.0f;
  uint8_t one = 0;
  const float w1 = 1.0f;
  CHECK(q4_quantize_row(nullptr, 1, &one, &s) == Q4_EINVAL);
  CHECK(q4_quantize_row(&w1, -1, &one, &s) == Q4_EINVAL);
  CHECK(q4_quantize_row(&w1, 1, nullptr, &s) == Q4_EINVAL);
  CHECK(q8_quantize_row(&w1, 1, nullptr, &s) == Q4_EINVAL);
}

static void pack(std::mt19937 &rng) {
  std::uniform_int_distribution<int> code(-8, 7);
  for (int64_t N : {0, 1, 3, 17}) {
    for (int64_t K : {0, 1, 2, 5, 4095, 4096, 4097}) {
      std::vector<int8_t> c(static_cast<size_t>(N * K + 1));
      for (auto &v : c) v = static_cast<int8_t>(code(rng));
      for (q4_enc enc : {Q4_ENC_TWOS, Q4_ENC_EXCESS8}) {
        Exact packed(static_cast<size_t>(N * ((K + 1) / 2)));
        CHECK(q4_pack(c.data(), N, K, enc, packed.p) == Q4_OK);
        for (int64_t n = 0; n < N; ++n)
          for (int64_t k = 0; k < K; ++k) {
            const unsigned u = (packed.p[n * ((K + 1) / 2) + k / 2] >> (4 * (k & 1))) & 0xF;
            const int q = enc == Q4_ENC_EXCESS8 ? static_cast<int>(u) - 8 : (u < 8 ? static_cast<int>(u) : static_cast<int>(u) - 16);
            CHECK(q == c[n * K + k]);
          }
      }
    }
  }
  // codes out of range, unknown encodings and N * K past int64: rejected, nothing written
  int8_t bad[4] = {0, 8, 0, 0};
  uint8_t out[2] = {0xA5, 0xA5};
  CHECK(q4_pack(bad, 1, 4, Q4_ENC_TWOS, out) == Q4_EINVAL);
  bad[1] = -9;
  CHECK(q4_pack(bad, 1, 4, Q4_ENC_EXCESS8, out) == Q4_EINVAL);
  bad[1] = 0;
  CHECK(q4_pack(bad, 1, 4, static_cast<q4_enc>(7), out) == Q4_EINVAL);
  CHECK(q4_pack(bad, INT64_MAX / 2, 4, Q4_ENC_TWOS, out) == Q4_EINVAL);
  CHECK(q4_pack(bad, -1, 4, Q4_ENC_TWOS, out) == Q4_EINVAL);
  CHECK(out[0] == 0xA5 && out[1] == 0xA5);
  for (int st = 0; st <= 5; ++st) CHECK(q4_status_string(static_cast<q4_status>(st)) != nullptr);
}

int main() {
  std::mt19937 rng(20261202);
  quantize_rows(rng);
  rejected_rows();
  pack(rng);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer checks ok\n");
  return 0;
}
