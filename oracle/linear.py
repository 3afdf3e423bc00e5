"""Oracle: the fused quantized linear y = x W^T (test infrastructure only).

Every function returns what the method computes for one call, from the
stored bytes, with no blocking, fusion or reordering beyond the definition.

Sources (page title, section):
  * "Fused int4 and int8 dequantize-matmul in C", section 2.3 (the factored
    sum): y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k], with
    g = floor(k / G); int8 is the same with one group per row.
  * same page, section 2.2: the shape rules (K even, G even and positive,
    K a multiple of G) and the f16 scale format.
  * ftts_kernels module int4, "Packing" and dot_i32_q4 / linear_q4: the
    int8-activation (W4A8) form, an exact integer dot product with the
    stored bias cancelled, and the scales applied once per output element.
  * ftts_kernels module int8, module head: exact i32 accumulation, then the
    two f32 scales applied once, after accumulation, in one fixed order.
  * "The 4-bit CPU path", section "W4A8": per-group zero points from the
    checkpoint in place of the synthesised constant 8 (the asymmetric
    layout, linear_w4a16_zp / linear_w4a8_zp).
  * "Fused int4 and int8 dequantize-matmul in C", sections 3 and 4, and
    ftts_kernels module int8, linear_w8a16: int8 weights with one scale per
    row against float activations (linear_w8a32 / linear_w8a16).

Precision:
  * Float-activation paths (W4A32, W4A16, W8A32, W8A16) return the float64
    value of the factored sum.  Each product x*q*s is exact in float64; the result is
    within K * 2**-53 * sum|x q s| of the exact real value.
  * Integer-activation paths (W4A8, W8A8) return float32 values defined
    operation by operation (each product and sum rounded to binary32):
      per channel:  y = (f32(acc) * s_x[m]) * s_w[n]
      grouped:      t = f32(acc_0) * s_0;  t = t + f32(acc_g) * s_g for
                    g = 1 .. K/G - 1 in increasing g;  y = t * s_x[m]
    The integer accumulators are exact: they are formed with a float64
    matrix product whose every product and partial sum is an integer below
    2**53, then checked to be integral.
"""
from __future__ import annotations

import numpy as np

from .formats import (EXCESS8, TWOS, bf16_bits_to_f32, f16_bits_to_float,
                      unpack_codes, unpack_nibbles)


def check_group_shape(K: int, G: int) -> None:
    """Shape rule of the grouped layout: K even, G even and > 0, G | K."""
    if K % 2 != 0 or G <= 0 or G % 2 != 0 or K % G != 0:
        raise ValueError(f"bad grouped shape K={K} G={G}")


def _exact_int_matmul(a, b):
    """a [M, K] int, b [N, K] int -> exact integer a @ b.T as int64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    bound = np.abs(a).max(initial=0) * np.abs(b).max(initial=0) * a.shape[1]
    if bound >= 2.0 ** 53:
        raise ValueError("integer accumulator would not be exact in float64")
    r = a @ b.T
    ri = np.rint(r)
    assert np.array_equal(r, ri)
    return ri.astype(np.int64)


def _grouped_float(xf64, codes, scales64, G):
    """sum_g s[n,g] * (sum_{k in g} x[m,k] q[n,k]) in float64."""
    M, K = xf64.shape
    N = codes.shape[0]
    y = np.zeros((M, N), np.float64)
    qf = codes.astype(np.float64)
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        partial = xf64[:, ks] @ qf[:, ks].T          # [M, N], this group only
        y += partial * scales64[None, :, g]
    return y


def linear_w4a32(x, qweight, scales_f16, G: int, enc: str = TWOS):
    """W4A32: f32 x [M, K], packed int4 [N, K/2], f16 bits [N, K/G] -> f64 [M, N]."""
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    check_group_shape(K, G)
    codes = unpack_codes(qweight, K, enc)
    s = f16_bits_to_float(scales_f16).reshape(codes.shape[0], K // G)
    return _grouped_float(x.astype(np.float64), codes, s, G)


def linear_w4a16(x_bf16, qweight, scales_bf16, G: int, enc: str = EXCESS8):
    """W4A16: bf16 bits x [M, K], packed int4, bf16 bits [N, K/G] -> f64 [M, N]."""
    xf = bf16_bits_to_f32(x_bf16).astype(np.float64)
    M, K = xf.shape
    check_group_shape(K, G)
    codes = unpack_codes(qweight, K, enc)
    s = bf16_bits_to_f32(scales_bf16).astype(np.float64).reshape(codes.shape[0], K // G)
    return _grouped_float(xf, codes, s, G)


def int_accumulators(xq, codes, G: int = 0):
    """Exact integer accumulators.

    G == 0: acc[m, n] = sum_k xq[m,k] q[n,k]            -> int64 [M, N]
    G  > 0: acc[m, n, g] = sum_{k in g} xq[m,k] q[n,k]  -> int64 [M, N, K/G]
    """
    xq = np.asarray(xq, dtype=np.int64)
    codes = np.asarray(codes, dtype=np.int64)
    if G == 0:
        return _exact_int_matmul(xq, codes)
    K = xq.shape[1]
    return np.stack([_exact_int_matmul(xq[:, g * G:(g + 1) * G], codes[:, g * G:(g + 1) * G])
                     for g in range(K // G)], axis=-1)


def epilogue_per_channel(acc, sx, sw):
    """y[m,n] = (f32(acc) * s_x[m]) * s_w[n], each product rounded to f32."""
    a = np.asarray(acc).astype(np.float32)
    sx = np.asarray(sx, dtype=np.float32)
    sw = np.asarray(sw, dtype=np.float32)
    t = (a * sx[:, None]).astype(np.float32)
    return (t * sw[None, :]).astype(np.float32)


def epilogue_grouped(acc_g, sx, sg):
    """t = f32(acc_0)*s_0; t += f32(acc_g)*s_g in increasing g; y = t*s_x[m].

    acc_g is [M, N, Gn]; sg is f32 [N, Gn].  Each product and each sum is
    rounded to f32 (an explicit loop over g, never a library reduction).
    """
    acc_g = np.asarray(acc_g)
    sg = np.asarray(sg, dtype=np.float32)
    sx = np.asarray(sx, dtype=np.float32)
    Gn = acc_g.shape[2]
    t = (acc_g[:, :, 0].astype(np.float32) * sg[None, :, 0]).astype(np.float32)
    for g in range(1, Gn):
        p = (acc_g[:, :, g].astype(np.float32) * sg[None, :, g]).astype(np.float32)
        t = (t + p).astype(np.float32)
    return (t * sx[:, None]).astype(np.float32)


def linear_w4a8(xq, sx, qweight, sw, G: int = 0, enc: str = EXCESS8):
    """W4A8: int8 xq [M, K] + f32 s_x [M], packed int4 [N, ceil(K/2)].

    G == 0: per-output-channel scale s_w f32 [N]; any K >= 0 (odd K uses the
            pad nibble, which decodes to 0).
    G  > 0: group scales f32 [N, K/G]; grouped shape rules apply.
    Returns f32 [M, N].
    """
    xq = np.asarray(xq, dtype=np.int8)
    M, K = xq.shape
    codes = unpack_codes(qweight, K, enc)
    if G == 0:
        acc = int_accumulators(xq, codes, 0)
        return epilogue_per_channel(acc, sx, np.asarray(sw, np.float32).reshape(-1))
    check_group_shape(K, G)
    acc_g = int_accumulators(xq, codes, G)
    return epilogue_grouped(acc_g, sx, np.asarray(sw, np.float32).reshape(codes.shape[0], K // G))


def codes_with_zero_points(qweight, zeros, K: int, G: int):
    """Asymmetric codes q[n,k] = u[n,k] - z[n, k // G] from the raw stored
    nibbles u (0..15) and one zero point z (0..15) per row and group.

    "The 4-bit CPU path", section "W4A8": a checkpoint's zero points are used
    where it has them, and the constant 8 is synthesised only otherwise, so a
    zero point takes the place of the 8 in u - 8; z = 8 everywhere is the
    symmetric excess-8 layout.
    """
    check_group_shape(K, G)
    u = unpack_nibbles(qweight, K)
    z = np.asarray(zeros, dtype=np.int64).reshape(u.shape[0], K // G)
    if np.any((z < 0) | (z > 15)):
        raise ValueError("a 4-bit zero point lies in 0..15")
    return u - np.repeat(z, G, axis=1)


def linear_w4a16_zp(x_bf16, qweight, scales_bf16, zeros, G: int):
    """W4A16 with per-group zero points: bf16 bits x [M, K], packed nibbles,
    bf16 bits scales [N, K/G], uint8 zero points [N, K/G] -> f64 [M, N]:
    y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] (u[n,k] - z[n,g])."""
    xf = bf16_bits_to_f32(x_bf16).astype(np.float64)
    M, K = xf.shape
    codes = codes_with_zero_points(qweight, zeros, K, G)
    s = bf16_bits_to_f32(scales_bf16).astype(np.float64).reshape(codes.shape[0], K // G)
    return _grouped_float(xf, codes, s, G)


def linear_w4a8_zp(xq, sx, qweight, sw, zeros, G: int):
    """Grouped W4A8 with per-group zero points: acc_g = sum_{k in g} xq q
    with q = u - z[n,g], exact; then the grouped f32 epilogue -> f32 [M, N]."""
    xq = np.asarray(xq, dtype=np.int8)
    M, K = xq.shape
    codes = codes_with_zero_points(qweight, zeros, K, G)
    acc_g = int_accumulators(xq, codes, G)
    return epilogue_grouped(acc_g, sx, np.asarray(sw, np.float32).reshape(codes.shape[0], K // G))


def linear_w8a8(xq, sx, wq, sw):
    """W8A8: int8 xq [M, K], int8 weights [N, K], f32 scales -> f32 [M, N]."""
    acc = int_accumulators(np.asarray(xq, np.int8), np.asarray(wq, np.int8), 0)
    return epilogue_per_channel(acc, sx, sw)


def _per_row_float(xf64, wq, sw):
    """y[m,n] = s[n] * sum_k x[m,k] q[n,k] in float64 (the one-scale-per-row
    factored sum)."""
    q = np.asarray(wq, dtype=np.int8).astype(np.float64)
    s = np.asarray(sw, dtype=np.float32).astype(np.float64).reshape(-1)
    return (xf64 @ q.T) * s[None, :]


def linear_w8a32(x, wq, sw):
    """W8A32 ("Fused int4 and int8 dequantize-matmul in C", section 4,
    tl_matmul_q8_f32): f32 x [M, K], int8 weights [N, K], f32 per-row
    scales [N] -> f64 [M, N]."""
    return _per_row_float(np.asarray(x, dtype=np.float32).astype(np.float64), wq, sw)


def linear_w8a16(x_bf16, wq, sw):
    """W8A16 (ftts_kernels module int8, linear_w8a16: float activations
    against a Q8 matrix, here bf16 as in the W4A16 layout): bf16 bits x
    [M, K], int8 weights [N, K], f32 per-row scales [N] -> f64 [M, N]."""
    return _per_row_float(bf16_bits_to_f32(x_bf16).astype(np.float64), wq, sw)


def linear_w4a8_dynamic(x, qweight, sw, G: int = 0, enc: str = EXCESS8, dtype: str = "f32"):
    """Quantize the activation rows (canonical Q8 recipe), then W4A8."""
    from .quantize import quantize_q8_rows
    xq, sx = quantize_q8_rows(x, dtype)
    return linear_w4a8(xq, sx, qweight, sw, G, enc), xq, sx


def dequantize_w4(qweight, scales64, K: int, G: int, enc: str):
    """The float64 weight matrix W[n,k] = q[n,k] * s[n, k // G] (for pins only)."""
    codes = unpack_codes(qweight, K, enc).astype(np.float64)
    return codes * np.repeat(np.asarray(scales64, np.float64), G, axis=1)


def abs_terms(x64, qweight, scales64, K: int, G: int, enc: str):
    """c[m,n] = sum_k |x[m,k] q[n,k] s[n,k//G]|, the condition scale of y[m,n]."""
    codes = np.abs(unpack_codes(qweight, K, enc)).astype(np.float64)
    return _grouped_float(np.abs(np.asarray(x64, np.float64)), codes,
                          np.abs(np.asarray(scales64, np.float64)), G)
