/*
 * q4_probe.h — diagnostics of libq4_probe, the ceilings the linear's
 * kernels are measured against on the running MI355X (gfx950): how fast a
 * plain kernel streams a buffer of a given size from memory, and how many
 * int8 matrix operations per second the matrix cores complete, with the
 * shader clock they ran at.  Not part of the linear itself; the benchmark
 * reports each kernel's time as a fraction of these.
 *
 * Device pointers, stream-ordered and asynchronous like libq4's device
 * calls ("Fused int4 and int8 dequantize-matmul in C", section 4: status
 * return, caller-owned buffers, nothing written on an error).
 */
#ifndef Q4_PROBE_H
#define Q4_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "q4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `buf` once with 16-byte nontemporal loads (the
 * decode kernels' access); sink[blocks] receives words that depend on the
 * data (their values have no meaning).  `blocks`
 * workgroups of `threads` threads (64, 128, 256 or 512) stride over the
 * buffer.  EINVAL: NULL, buf not 16-byte aligned, bytes not a multiple of
 * 16 or zero, blocks outside 1..65535, other thread counts, sink
 * overlapping buf. */
q4_status q4_probe_read(const void *buf, size_t bytes, uint32_t *sink, int64_t blocks, int64_t threads,
                        void *stream);

/* Matrix-core rate: `blocks` workgroups of 256 threads (one wave per SIMD
 * when one workgroup runs per CU), each wave issuing `iters` rounds of 16
 * independent v_mfma_i32_32x32x32_i8 (four accumulation chains), i.e.
 * iters * 16 * 32768 multiply-adds per wave.  out[4 * blocks * 2] u64: per
 * wave, the shader-clock cycles (s_memtime) and the 100 MHz reference
 * ticks (s_memrealtime) it ran for, so the shader clock is
 * cycles / ticks * 100 MHz.  EINVAL: NULL, blocks outside 1..65535, iters
 * outside 1..1000000. */
q4_status q4_probe_mfma_i8(uint64_t *out, int64_t blocks, int64_t iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_PROBE_H */
