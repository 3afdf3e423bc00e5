// Internal launchers of libq4's kernels.  Callers (q4_api.hip) have already
// validated every argument; the launchers only choose grid shapes and
// enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

// Is the current device gfx950?  (Cached per device; the API checks it
// before every launch.)
bool device_is_gfx950();

// Stored-nibble encodings, as in q4_enc.
enum Enc : int { kTwos = 0, kExcess8 = 1 };

// y[0..n) = 0 for float outputs, written by a kernel (no memset node, so a
// captured graph replays it like any other kernel).
hipError_t launch_zero(void *p, size_t bytes, hipStream_t st);

// Activation rows -> int8 codes + f32 scales (canonical Q8 recipe).
hipError_t launch_quantize_rows(const void *x, bool x_bf16, int64_t M, int64_t K, int8_t *xq,
                                float *sx, hipStream_t st);

// General kernels: any shape the API accepts, byte-granular loads.
// Float activations (W4A32: f32 x, f16 scales; W4A16: bf16 x, bf16 scales).
// zp (optional, W4A16 and grouped W4A8): uint8 zero points [N, K/G]; then
// a weight is s * (u - z) with u the stored nibble, and enc is not used.
hipError_t launch_generic_float(const void *x, bool x_bf16, const uint8_t *wq, const uint16_t *s,
                                bool s_bf16, float *yf, uint16_t *yb, int64_t M, int64_t N,
                                int64_t K, int64_t G, int enc, hipStream_t st,
                                const uint8_t *zp = nullptr);
// Integer activations (W4A8 per channel / grouped, W8A8).
hipError_t launch_generic_int(const int8_t *xq, const float *sx, const void *w, bool w_int8,
                              const float *sw, float *y, int64_t M, int64_t N, int64_t K,
                              int64_t G, int enc, hipStream_t st, const uint8_t *zp = nullptr);

// int8 weights, one f32 scale per row, f32 or bf16 activations (W8A32 /
// W8A16): y = s[n] * sum_k x q; yf and / or yb (bf16 RNE) written.
hipError_t launch_generic_w8_float(const void *x, bool x_bf16, const int8_t *wq, const float *s, float *yf,
                                   uint16_t *yb, int64_t M, int64_t N, int64_t K, hipStream_t st);
bool gemv_stream_w8_ok(const void *x, const void *wq, int64_t M, int64_t K);
hipError_t launch_gemv_stream_w8(const void *x, bool x_bf16, const int8_t *wq, const float *s, float *yf,
                                 uint16_t *yb, int64_t M, int64_t N, int64_t K, hipStream_t st);

// W4A32 on the vector ALUs: f32 x, f16 group scales, G a multiple of 32,
// 16-byte aligned x and wq; every M (workgroups of 1 or 2 activation rows).
bool gemv_stream_w4a32_ok(const void *x, const void *wq, int64_t M, int64_t K, int64_t G);
hipError_t launch_gemv_stream_w4a32(const float *x, const uint8_t *wq, const uint16_t *s, float *y, int64_t M,
                                    int64_t N, int64_t K, int64_t G, int enc, hipStream_t st);

// Decode GEMV on MFMA (M in blocks of 16).  *_ok says whether the fast
// kernel serves a shape / alignment; the launcher must only be called then.
bool gemv_w4a16_ok(const void *x, const void *wq, int64_t K, int64_t G);
hipError_t launch_gemv_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                             uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                             hipStream_t st, const uint8_t *zp = nullptr);
// Decode GEMV for W4A16 on the matrix cores (M <= 16, G a multiple of 128).
bool gemv_mc_w4a16_ok(const void *x, const void *wq, int64_t M, int64_t K, int64_t G);
hipError_t launch_gemv_mc_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                                uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                                hipStream_t st);
// Decode GEMV for W4A16 on the vector ALUs (M <= 16, K and G multiples of 32).
bool gemv_stream_w4a16_ok(const void *x, const void *wq, int64_t M, int64_t K, int64_t G);
hipError_t launch_gemv_stream_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                                    uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                                    hipStream_t st, const uint8_t *zp = nullptr);
// Decode GEMV for per-channel W4A8 on the vector ALUs (M <= 16, ceil(K/2) a
// multiple of 16).  xt: 0 = int8 codes with scales sx, 1 = f32 x, 2 = bf16 x
// (quantized inside with the Q8 recipe; sx unused).
bool gemv_chan_w4a8_ok(const void *wq, int64_t M, int64_t K);
hipError_t launch_gemv_chan_w4a8(const void *x, int xt, const float *sx, const uint8_t *wq,
                                 const float *sw, float *y, int64_t M, int64_t N, int64_t K, int enc,
                                 hipStream_t st);
// The same kernel over several independent problems in one launch (float
// x quantized inside, excess-8 weights, one M <= 16 for all).  The caller
// lists only problems with N > 0 and K > 0 that gemv_chan_w4a8_ok accepts,
// at most gemv_chan_w4a8_multi_max() of them, whose tiles of 16 weight rows
// (gemv_chan_w4a8_multi_tiles(N) each) sum to at most 2^24 - 1.
struct ChanProblem {
  const void *x;
  const uint8_t *wq;
  const float *sw;
  float *y;
  int64_t N, K;
};
int64_t gemv_chan_w4a8_multi_max();
int64_t gemv_chan_w4a8_multi_tiles(int64_t N);
hipError_t launch_gemv_chan_w4a8_multi(const ChanProblem *pr, int count, int64_t M, bool x_bf16,
                                       hipStream_t st);
bool gemv_w4a8_ok(const void *wq, int64_t K, int64_t G);
hipError_t launch_gemv_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                            float *y, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                            hipStream_t st, const uint8_t *zp = nullptr);
// Dynamic W4A8 in one launch: f32 or bf16 activation rows quantized inside
// the MFMA GEMV (a small activation matrix).
bool gemv_w4a8_fused_ok(const void *wq, int64_t M, int64_t K, int64_t G, bool x_bf16);
hipError_t launch_gemv_w4a8_fused(const void *x, bool x_bf16, const uint8_t *wq, const float *sw, float *y,
                                  int64_t M, int64_t N, int64_t K, int64_t G, int enc, hipStream_t st,
                                  const uint8_t *zp = nullptr);
bool gemv_w8a8_ok(const void *wq, int64_t K);
hipError_t launch_gemv_w8a8(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw,
                            float *y, int64_t M, int64_t N, int64_t K, hipStream_t st);

// Prefill: LDS-tiled MFMA GEMM (M >= 17).
int device_cu_count();   // compute units of the current device, 0 if unknown
void tiled_w4a8_pieces(int64_t M, int64_t N, int cus, int *full, int *split, int64_t *tiles);
void tiled_w4a16_pieces(int64_t M, int64_t N, int cus, int *full, int64_t *pieces);
bool tiled_w4a8_ok(const void *xq, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G);
hipError_t launch_tiled_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                             float *y, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                             hipStream_t st, const uint8_t *zp = nullptr);
bool tiled_w4a16_ok(const void *x, const void *wq, int64_t M, int64_t N, int64_t K, int64_t G);
hipError_t launch_tiled_w4a16(const uint16_t *x, const uint8_t *wq, const uint16_t *s, float *yf,
                              uint16_t *yb, int64_t M, int64_t N, int64_t K, int64_t G, int enc,
                              hipStream_t st, const uint8_t *zp = nullptr);

}  // namespace q4
