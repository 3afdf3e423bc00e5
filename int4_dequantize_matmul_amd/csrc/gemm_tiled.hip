// Prefill: LDS-tiled MFMA GEMM (placeholder until the tiled kernels land;
// the dispatcher falls back to the decode kernels in blocks of 16 rows).
#include "kernels.hpp"

namespace q4 {

bool tiled_w4a8_ok(const void *, const void *, int64_t, int64_t, int64_t, int64_t) { return false; }
hipError_t launch_tiled_w4a8(const int8_t *, const float *, const uint8_t *, const float *, float *,
                             int64_t, int64_t, int64_t, int64_t, int, hipStream_t) {
  return hipErrorInvalidValue;
}
bool tiled_w4a16_ok(const void *, const void *, int64_t, int64_t, int64_t, int64_t) { return false; }
hipError_t launch_tiled_w4a16(const uint16_t *, const uint8_t *, const uint16_t *, float *, uint16_t *,
                              int64_t, int64_t, int64_t, int64_t, int, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace q4
