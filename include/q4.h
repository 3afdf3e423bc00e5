/*
 * q4.h — C ABI of libq4, the fused packed-int4 quantized linear y = x W^T
 * for AMD Instinct MI355X (gfx950).  W is never materialised in floating
 * point: each kernel reads the packed nibbles and applies the scales on the
 * fly.
 *
 * Definitions follow the reference pages (cited by page title and section):
 *   [tinyllm]  "Fused int4 and int8 dequantize-matmul in C"
 *   [int4]     ftts_kernels module int4 (docs.rs)
 *   [int8]     ftts_kernels module int8 (docs.rs)
 *   [cpu4bit]  "The 4-bit CPU path" (vllm-omni edge documentation)
 *
 * Conventions shared by every call
 *   - Row-major, contiguous buffers; no strides.  x is [M, K], W is [N, K]
 *     (the Linear's [out, in]), y is [M, N].
 *   - Packed weights: uint8 [N, ceil(K/2)]; byte b of row n holds column 2b
 *     in bits 0-3 and column 2b+1 in bits 4-7 ([tinyllm] section 2.2,
 *     [int4] "Packing").
 *   - Nibble encodings (q4_enc): two's complement, u < 8 ? u : u - 16
 *     ([tinyllm] section 2.2); or excess-8, u - 8 ([int4] "Packing").
 *   - Device calls take DEVICE pointers and a hipStream_t passed as void*
 *     (NULL = the null stream).  They validate every argument on the host
 *     before any HIP call, enqueue on that stream and return; results are
 *     ready after the caller synchronises the stream.  The library
 *     allocates nothing and keeps no pointer after a call returns.
 *   - Check order ([tinyllm] section 4): Q4_EINVAL (negative dimension, NULL
 *     pointer, unknown enum, output overlapping an input, workspace too
 *     small), then Q4_ESHAPE (shape rules), then M == 0 or N == 0 is a
 *     no-op returning Q4_OK, and K == 0 sets y to 0.  On any error nothing
 *     is read or written.  NULL is Q4_EINVAL even when a dimension is 0.
 *   - Q4_EDEVICE: the current device is not gfx950, or a launch failed.
 *     Faults inside a kernel surface at the caller's stream synchronise.
 *   - Integer-activation calls (W4A8, W8A8) are bit-exact: i32 accumulators
 *     and a fixed order of f32 scale multiplications without FMA.  Float
 *     calls (W4A32, W4A16, W8A32, W8A16) are accurate to 1e-5 (f32 out) or
 *     2e-2 (bf16 out) relative to max|y| against the exact value.
 *   - Thread safety: every call is reentrant; q4_set_path is a process-wide
 *     setting meant for tests and benchmarks.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  Q4_OK = 0,
  Q4_EINVAL = 1,  /* bad argument: NULL, negative dim, unknown enum, overlap */
  Q4_ESHAPE = 2,  /* shape rule broken (K, G) or a size beyond the limits  */
  Q4_EDEVICE = 3,  /* not a gfx950 device, or a HIP launch error           */
  Q4_EMISMATCH = 4 /* q4_selftest: a kernel result differed from its closed form */
} q4_status;

typedef enum {
  Q4_ENC_TWOS = 0,    /* stored u means u if u < 8, else u - 16 */
  Q4_ENC_EXCESS8 = 1  /* stored u means u - 8                   */
} q4_enc;

typedef enum {
  Q4_DT_F32 = 0,      /* IEEE binary32                                  */
  Q4_DT_BF16 = 1      /* bfloat16 bit patterns (top half of a binary32) */
} q4_dtype;

typedef enum {
  Q4_PATH_AUTO = 0,     /* the measured plan (q4_route_plan): decode kernels up
                         * to a per-shape batch size (16 rows at N >= 13312, up
                         * to 96 at N = K = 2048), tiled MFMA above where the
                         * shape allows it, the general kernels otherwise;
                         * per-channel W4A8 takes its streaming kernel at
                         * M = 1 and the MFMA GEMV from M = 2                   */
  Q4_PATH_GENERIC = 1,  /* the general kernels (any valid shape)                 */
  Q4_PATH_GEMV = 2,     /* the decode kernels                                    */
  Q4_PATH_TILED = 3,    /* the LDS-tiled MFMA kernels, where a shape allows      */
  Q4_PATH_GEMV_MC = 4   /* W4A16 decode on the matrix cores (G of 128, 256 or
                         * 512, M <= 16): one kernel for every batch size, so
                         * still batch-invariant, and faster than the default
                         * decode kernel from about 4 rows up.  Other calls
                         * treat it as Q4_PATH_GEMV.                             */
} q4_path;

/* Largest K for which the i32 accumulators provably cannot overflow
 * (|x| <= 128 and a stored nibble <= 15, or |w| <= 128 for int8 weights);
 * larger K is Q4_ESHAPE ([int8] "Tier law": the reduction must fit i32). */
#define Q4_W4A8_MAX_K 1048576
#define Q4_W8A8_MAX_K 131071

/* ------------------------------------------------------------------------
 * Host calls (host pointers; plain C++, IEEE binary32, no device needed).
 * ---------------------------------------------------------------------- */

/* Quantize one weight row ([int4] "The quantization contract", "Packing"):
 * a = max|w|; scale = a / 7 (correctly rounded); q = clamp(rint(w / scale),
 * -7, 7) with ties to even; stored as q + 8 two per byte, low nibble first;
 * an odd K pads the last high nibble with 8.  An all-zero row gives scale 0
 * and codes 0.  w: [K] floats; packed: ceil(K/2) bytes written; *scale
 * written.  EINVAL for NULL, K < 0 or a non-finite input (nothing written). */
q4_status q4_quantize_row(const float *w, int64_t K, uint8_t *packed, float *scale);

/* Quantize one row with the canonical Q8 recipe ([int8] quantize_row_q8):
 * scale = max|x| / 127, q = clamp(rint(x / scale), -127, 127), ties to even;
 * -128 is never emitted.  q: [K] int8 written; *scale written. */
q4_status q8_quantize_row(const float *x, int64_t K, int8_t *q, float *scale);

/* Pack int codes [N, K] (each in [-8, 7]) into [N, ceil(K/2)] bytes in the
 * given encoding; the odd-K pad nibble is the encoding's zero (8 or 0).
 * EINVAL for a code out of range (nothing written). */
q4_status q4_pack(const int8_t *codes, int64_t N, int64_t K, q4_enc enc, uint8_t *packed);

/* ------------------------------------------------------------------------
 * Device calls (device pointers, stream-ordered, asynchronous).
 * ---------------------------------------------------------------------- */

/* Quantize activation rows with the Q8 recipe ([int8] module head:
 * activations quantized dynamically per row).  x: [M, K] f32 or bf16 (xt);
 * xq: [M, K] int8 out; sx: [M] f32 scales out.  bf16 is widened exactly to
 * f32 first.  A row of zeros gives scale 0 and codes 0.  Non-finite input
 * gives undefined codes. */
q4_status q8_quantize_rows(const void *x, q4_dtype xt, int64_t M, int64_t K,
                           int8_t *xq, float *sx, void *stream);

/* W4A32 ([tinyllm] sections 2.3, 4): y[m,n] = sum_g s[n,g] sum_{k in g}
 * x[m,k] q[n,k].  x: f32 [M, K]; wq: [N, K/2]; scales_f16: IEEE half bit
 * patterns [N, K/G] (subnormals honoured); y: f32 [M, N].
 * ESHAPE: K odd, G odd or <= 0, K % G != 0.  One decode kernel serves
 * every M when G is a multiple of 32 and x and wq are 16-byte aligned (a
 * row's bits then do not depend on M); other calls take the general
 * kernel. */
q4_status q4_linear_w4a32(const float *x, const uint8_t *wq, const uint16_t *scales_f16,
                          float *y, int64_t M, int64_t N, int64_t K, int64_t G,
                          q4_enc enc, void *stream);

/* W4A16: the same factored sum with bf16 activations and bf16 group scales,
 * accumulated in f32.  x_bf16: [M, K]; scales_bf16: [N, K/G]; y_bf16: [M, N]
 * bf16 rounded to nearest even from the f32 result (required); y_f32: the
 * f32 result [M, N] (optional, NULL = not written).  ESHAPE as W4A32. */
q4_status q4_linear_w4a16(const uint16_t *x_bf16, const uint8_t *wq, const uint16_t *scales_bf16,
                          uint16_t *y_bf16, float *y_f32, int64_t M, int64_t N, int64_t K,
                          int64_t G, q4_enc enc, void *stream);

/* W4A8 ([int4] dot_i32_q4, linear_q4; [int8] module head): int8 activations
 * xq [M, K] with f32 row scales sx [M]; packed int4 wq [N, ceil(K/2)].
 *   G == 0, per output channel: sw f32 [N]; any K >= 0 (odd K reads the pad
 *     nibble, which meets a zero activation);
 *     acc = sum_k xq q (exact i32); y = (f32(acc) * sx[m]) * sw[n].
 *   G  > 0, grouped: sw f32 [N, K/G]; ESHAPE rules as W4A32;
 *     t = f32(acc_0) s_0; t = t + f32(acc_g) s_g for g = 1.. in increasing
 *     g; y = t * sx[m]  (every product and sum rounded to f32, no FMA).
 * y: f32 [M, N].  ESHAPE also for K > Q4_W4A8_MAX_K. */
q4_status q4_linear_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                         float *y, int64_t M, int64_t N, int64_t K, int64_t G, q4_enc enc,
                         void *stream);

/* Asymmetric layouts with per-group zero points ([cpu4bit] section "W4A8":
 * a checkpoint's zero points are used where present, and the constant 8 is
 * synthesised only otherwise).  The stored nibble u (0..15) is used as is
 * and a weight is s[n,g] * (u[n,k] - z[n,g]), g = k / G, with zeros a
 * uint8 array [N, K/G] of 4-bit zero points (0..15; larger values are not
 * checked on the device and give unspecified results).  z = 8 everywhere
 * reproduces the symmetric excess-8 call exactly.  Checks and the result
 * contract are those of the symmetric call; zeros is one more input
 * (NULL is EINVAL, an overlap with an output is EINVAL).
 *
 * W4A16: as q4_linear_w4a16 (same shape rules and tolerance).  The
 * matrix-core decode route (Q4_PATH_GEMV_MC) does not take zero points;
 * such calls run the default decode kernels. */
q4_status q4_linear_w4a16_zp(const uint16_t *x_bf16, const uint8_t *wq, const uint16_t *scales_bf16,
                             const uint8_t *zeros, uint16_t *y_bf16, float *y_f32, int64_t M,
                             int64_t N, int64_t K, int64_t G, void *stream);

/* Grouped W4A8 (G > 0; G == 0 is ESHAPE): acc_g = sum_{k in g} xq (u - z)
 * exactly in i32, then the grouped epilogue of q4_linear_w4a8, bit for bit,
 * on the same routes as the symmetric call. */
q4_status q4_linear_w4a8_zp(const int8_t *xq, const float *sx, const uint8_t *wq, const float *sw,
                            const uint8_t *zeros, float *y, int64_t M, int64_t N, int64_t K,
                            int64_t G, void *stream);

/* Bytes of device workspace q4_linear_w4a8_dynamic needs for M rows of K:
 * room for xq [M, K] and sx [M], each 256-byte aligned. */
size_t q4_w4a8_dynamic_workspace(int64_t M, int64_t K);

/* Dynamic W4A8 ([int8] linear_q8_dynamic): q8_quantize_rows of x into the
 * caller's workspace ws (ws_bytes >= q4_w4a8_dynamic_workspace(M, K), device
 * memory, 256-byte aligned), then q4_linear_w4a8.  Per-channel decode of
 * one row (G == 0, M == 1; every M <= 16 on the forced decode route)
 * quantizes inside the GEMV instead, with the same codes, and leaves ws
 * untouched; its contents after any call are unspecified.
 * EINVAL for a small or misaligned workspace or one overlapping another
 * buffer. */
q4_status q4_linear_w4a8_dynamic(const void *x, q4_dtype xt, const uint8_t *wq, const float *sw,
                                 float *y, int64_t M, int64_t N, int64_t K, int64_t G,
                                 q4_enc enc, void *ws, size_t ws_bytes, void *stream);

/* Largest workspace q4_linear_w4a8_dynamic_noalloc serves from the
 * library's own device array (q4_w4a8_dynamic_workspace(M, K) must not
 * exceed it): 8 MiB, for example up to 4088 rows of K = 2048 or 1024 rows
 * of K = 8184. */
#define Q4_NOALLOC_SCRATCH_BYTES 8388608

/* For callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as q4_linear_w4a8_dynamic, bit for bit on the same route, with the
 * activation codes and scales in a scratch array the library holds on each
 * device (Q4_NOALLOC_SCRATCH_BYTES, kept until the process ends) instead of
 * a caller workspace.  The caller passes x, wq, sw and y as before; the call
 * allocates nothing.  Checks as q4_linear_w4a8_dynamic without the
 * workspace ones, then Q4_ESHAPE if q4_w4a8_dynamic_workspace(M, K) exceeds
 * Q4_NOALLOC_SCRATCH_BYTES; Q4_EDEVICE if the array's address cannot be
 * found on the current device.  Every call on one device shares that
 * device's array: calls that may run at the same time on one device (two
 * streams, or two host threads) race and give undefined results; calls
 * ordered on one stream do not.  Nothing in the array needs to start at
 * zero: each call writes the codes and scales it reads. */
q4_status q4_linear_w4a8_dynamic_noalloc(const void *x, q4_dtype xt, const uint8_t *wq, const float *sw,
                                         float *y, int64_t M, int64_t N, int64_t K, int64_t G,
                                         q4_enc enc, void *stream);

/* One per-channel linear of q4_linear_w4a8_dynamic_multi (device pointers):
 * x [M, K] f32 or bf16, wq [N, ceil(K/2)] excess-8 nibbles (16-byte
 * aligned), sw [N], y [M, N] f32. */
typedef struct {
  const void *x;
  const uint8_t *wq;
  const float *sw;
  float *y;
  int64_t N, K;
} q4_w4a8_problem;

#define Q4_MULTI_MAX 64

/* Up to Q4_MULTI_MAX independent per-channel dynamic W4A8 linears
 * ([int8] linear_q8_dynamic; [int4] linear_q4) in one launch, for decode
 * steps that run many small linears (the microdecoder of [int4] "Why the
 * microdecoder, and why now" re-reads its five-layer body many times per
 * frame), where a launch per linear costs more than its weights take to
 * stream.  Every problem shares M
 * (0..16) and the activation type xt; each is quantized per row with the
 * Q8 recipe inside the kernel and computed exactly as a single
 * q4_linear_w4a8_dynamic call with G == 0 and Q4_ENC_EXCESS8 would compute
 * it, bit for bit.  problems is a HOST array, read before the call returns.
 * Checks: EINVAL for count < 0 or > Q4_MULTI_MAX, problems NULL with
 * count > 0, an unknown xt, M < 0, a NULL pointer or negative dimension in
 * any problem, wq not 16-byte aligned, or any y overlapping any input or
 * another y; ESHAPE for M > 16, K > Q4_W4A8_MAX_K, ceil(K/2) not a
 * multiple of 16 (for K > 0), activation codes beyond the 64 KB of LDS a
 * workgroup stages them in (2 KB per row of M, rounded up to a power of
 * two, per 2048 columns: K <= 63488 at M = 1, K <= 2048 at M = 16), or more
 * than 2^24 - 1 tiles of 16 weight rows in all.
 * Problems with N == 0 are skipped; K == 0 sets that y to 0.  count == 0 or
 * M == 0 is a no-op.  The call allocates nothing and launches one kernel
 * (plus one fill per problem with K == 0). */
q4_status q4_linear_w4a8_dynamic_multi(const q4_w4a8_problem *problems, int64_t count, q4_dtype xt,
                                       int64_t M, void *stream);

/* W8A8 ([int8] linear_q8, [tinyllm] section 2.3 int8 form): int8 xq [M, K]
 * with sx [M], int8 weights wq [N, K] with per-row sw [N];
 * y = (f32(acc) * sx[m]) * sw[n].  ESHAPE for K > Q4_W8A8_MAX_K. */
q4_status q8_linear_w8a8(const int8_t *xq, const float *sx, const int8_t *wq, const float *sw,
                         float *y, int64_t M, int64_t N, int64_t K, void *stream);

/* W8A32 ([tinyllm] section 4, tl_matmul_q8_f32; the int8 form of the worked
 * example in section 3): f32 x [M, K], int8 weights wq [N, K] (codes
 * -128..127) with one f32 scale per row sw [N]; y f32 [M, N] =
 * sw[n] * sum_k x[m,k] wq[n,k], accumulated in f32 (accurate to 1e-5
 * relative to max|y|).  Any K >= 0; K == 0 sets y = 0. */
q4_status q8_linear_w8a32(const float *x, const int8_t *wq, const float *sw, float *y,
                          int64_t M, int64_t N, int64_t K, void *stream);

/* W8A16 ([int8] linear_w8a16, float activations against a Q8 matrix; bf16
 * activations as in q4_linear_w4a16): bf16 x [M, K], int8 wq [N, K], f32
 * sw [N]; y_bf16 [M, N] (required) is the f32 result rounded to nearest
 * even, y_f32 (optional, may be NULL) the f32 result.  One decode kernel
 * serves every batch size, so a row's bits do not depend on M; there is no
 * tiled int8-weight kernel. */
q4_status q8_linear_w8a16(const uint16_t *x_bf16, const int8_t *wq, const float *sw, uint16_t *y_bf16,
                          float *y_f32, int64_t M, int64_t N, int64_t K, void *stream);

/* Process-wide route override for A/B tests and benchmarks ([int8] "Tier
 * law": routes are chosen by measurement and can be forced).  A forced route
 * that cannot serve a shape falls back to the generic kernels.  EINVAL for
 * an unknown value. */
q4_status q4_set_path(q4_path path);
q4_path q4_get_path(void);

/* Which kernel family the last successful device call on this thread used
 * (a q4_path value other than AUTO), for tests of the dispatcher. */
q4_path q4_last_path(void);

/* Operations whose route q4_route_plan reports. */
typedef enum {
  Q4_OP_W4A32 = 0,    /* q4_linear_w4a32                                   */
  Q4_OP_W4A16 = 1,    /* q4_linear_w4a16 (enc EXCESS8 or TWOS alike)        */
  Q4_OP_W4A16_ZP = 2, /* q4_linear_w4a16_zp                                */
  Q4_OP_W4A8 = 3,     /* q4_linear_w4a8 and the dynamic calls (G 0 or > 0) */
  Q4_OP_W4A8_ZP = 4,  /* q4_linear_w4a8_zp                                 */
  Q4_OP_W8A8 = 5      /* q8_linear_w8a8                                    */
} q4_op;

typedef struct {
  q4_path path;        /* the route; Q4_PATH_AUTO when nothing is launched
                        * (M or N zero); GENERIC for K == 0 (a fill)          */
  int32_t decode_max;  /* largest M this N and K send to a decode kernel on
                        * the AUTO route (INT32_MAX: the op has no tiled
                        * kernel)                                            */
  int32_t whole_tiles; /* tiled route: workgroups that own a whole 128-row
                        * tile                                               */
  int32_t piece_rows;  /* tiled route: rows of each remaining piece, 64 or
                        * 32 (32 for W4A8 only); 0 when every tile is whole  */
  int32_t pieces;      /* tiled route: workgroups of piece_rows rows         */
} q4_plan;

/* The route a call of this shape takes under the current q4_set_path
 * setting, when its device buffers are 16-byte aligned ([int8] Structs and
 * "Tier law": the kernel plan of a shape is decided by measurement).  Host
 * only: nothing runs on the device.  cus: compute units to plan the tiled
 * work split for, or 0 for the current device's (Q4_EDEVICE without a
 * gfx950 device).  EINVAL: plan NULL, unknown op, negative size or cus, or
 * G < 0; ESHAPE: the shape rules of the op's call.  The crossing from
 * decode to tiled was measured per shape (hot weights, G = 128) and a shape
 * takes the one of the measured shape nearest to it in (log N, log K). */
q4_status q4_route_plan(q4_op op, int64_t M, int64_t N, int64_t K, int64_t G, int32_t cus, q4_plan *plan);

/* Bytes of device workspace q4_selftest needs (about 12.5 MiB). */
size_t q4_selftest_workspace(void);

/* All-extreme proof rows through every kernel route on the current device
 * ([int8] "Tier law": every tier must equal the scalar definition exactly,
 * and a selftest runs the all-extreme rows through the real kernels on the
 * running silicon).  Activation codes +-127 against weight codes +7, -7, -8
 * (int8 weights +127, -127, -128) for W4A8 per channel and grouped (the
 * general kernels, the streaming and MFMA decode GEMVs, the tiled GEMM),
 * the fused activation quantizer and W8A8, at K = 1023, 2048, 5632, 131072
 * and the largest K each route accepts (Q4_W4A8_MAX_K, Q4_W8A8_MAX_K);
 * every output must equal its closed form bit for bit, which also shows
 * that no accumulator overflows.  ws: caller-owned device memory of at
 * least q4_selftest_workspace() bytes, 256-byte aligned (EINVAL
 * otherwise); its contents afterwards are unspecified.  Synchronises the
 * stream; takes milliseconds.  Q4_OK when every check passes, Q4_EMISMATCH
 * on the first wrong output, Q4_EDEVICE on a HIP error; q4_selftest_report
 * then describes the result. */
q4_status q4_selftest(void *ws, size_t ws_bytes, void *stream);

/* What the last q4_selftest on this thread found (the failing case and
 * value, or the number of checks passed); never NULL. */
const char *q4_selftest_report(void);

/* Static description of a status code; never NULL. */
const char *q4_status_string(q4_status st);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
