"""Oracle: the symmetric row quantizers (test infrastructure only).

Sources (page title, section):
  * ftts_kernels module int8, module head and quantize_row_q8: the canonical
    symmetric recipe, scale = max|row| / 127, round half to even, codes in
    [-127, 127], -128 never emitted; used for weight rows and, dynamically,
    for activation rows.
  * ftts_kernels module int4, "The quantization contract": the Q4 recipe has
    the same shape with 7 and [-7, 7] (-8 never emitted), per output channel.
  * ftts_kernels module int4, "Packing": store q + 8, low nibble first; an odd
    row pads its last high nibble with 8.

Arithmetic is IEEE binary32 throughout, as the pages fix f32 scales: the
scale is the correctly rounded quotient max|row| / qmax, each code is the
correctly rounded quotient w / scale rounded half-to-even and clamped.

Readings where the pages are silent: an all-zero row (or one whose scale
underflows to 0) gets scale 0 and all codes 0; non-finite input is rejected.
"""
from __future__ import annotations

import numpy as np

from .formats import EXCESS8, bf16_bits_to_f32, pack_codes


def _symmetric_row(w, qmax: int):
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 1:
        raise ValueError("one row at a time")
    if not np.all(np.isfinite(w)):
        raise ValueError("finite values only")
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(qmax))
    if scale == np.float32(0.0):
        return np.zeros(w.shape, np.int64), np.float32(0.0)
    ratio = (w / scale).astype(np.float32)       # f32 division per element
    q = np.rint(ratio)                            # half to even
    q = np.clip(q, -qmax, qmax).astype(np.int64)
    return q, scale


def quantize_q8_row(x):
    """One row -> (int8 codes [K], f32 scale): scale = max|x|/127."""
    q, s = _symmetric_row(x, 127)
    return q.astype(np.int8), s


def quantize_q4_codes_row(w):
    """One row -> (int codes in [-7, 7] [K], f32 scale): scale = max|w|/7."""
    return _symmetric_row(w, 7)


def quantize_q4_row(w):
    """One weight row -> (packed uint8 [ceil(K/2)], f32 scale), excess-8."""
    q, s = quantize_q4_codes_row(w)
    return pack_codes(q[None, :], EXCESS8)[0], s


def quantize_q4_matrix(W):
    """Rows of W [N, K] -> (packed uint8 [N, ceil(K/2)], f32 scales [N])."""
    W = np.asarray(W, dtype=np.float32)
    packed = []
    scales = np.empty(W.shape[0], np.float32)
    for n in range(W.shape[0]):
        p, scales[n] = quantize_q4_row(W[n])
        packed.append(p)
    K = W.shape[1]
    return (np.stack(packed) if packed else np.zeros((0, (K + 1) // 2), np.uint8)), scales


def quantize_q8_rows(x, dtype: str = "f32"):
    """Activation rows [M, K] -> (int8 [M, K], f32 scales [M]).

    dtype "bf16" means x holds bf16 bit patterns, widened exactly to f32
    before quantizing.
    """
    if dtype == "bf16":
        xf = bf16_bits_to_f32(x)
    elif dtype == "f32":
        xf = np.asarray(x, dtype=np.float32)
    else:
        raise ValueError(dtype)
    M, K = xf.shape
    xq = np.zeros((M, K), np.int8)
    sx = np.zeros(M, np.float32)
    for m in range(M):
        xq[m], sx[m] = quantize_q8_row(xf[m])
    return xq, sx
