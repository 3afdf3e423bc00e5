"""Oracle: storage formats of the packed-int4 linear (test infrastructure only).

Plain, slow, obviously correct CPU definitions of how codes and scales are
stored.  Only tests, the smoke check and the CPU-baseline leg of the bench use
this package; the product path never imports it.

Sources (page title, section):
  * "Fused int4 and int8 dequantize-matmul in C", section 2.2 "The int4 layout":
    qweight is uint8 [N, K/2]; byte b of row n keeps column 2b in bits 0-3 and
    column 2b+1 in bits 4-7; each nibble is a 4-bit two's-complement code
    (u < 8 means u, otherwise u - 16); scales are raw IEEE half bit patterns.
  * ftts_kernels module int4, "Packing": two nibbles per byte, low nibble
    first, along k; codes stored biased by +8 so [-7, 7] becomes [1, 15] and
    decoding is u - 8; an odd-length row pads its last high nibble with the
    biased zero 8.
  * The 16-bit brain-float format of the bf16 activations and scales is the
    top half of an IEEE binary32 pattern; its round-to-nearest-even encoding
    of an f32 value is written out below from that definition.
"""
from __future__ import annotations

import numpy as np

TWOS = "twos"        # two's-complement nibble, tinyllm layout
EXCESS8 = "excess8"  # nibble biased by +8, ftts int4 layout
ENCODINGS = (TWOS, EXCESS8)


def nibble_to_code(u, enc: str) -> np.ndarray:
    """Decode 4-bit stored values u in [0, 15] to signed codes.

    two's complement: u if u < 8 else u - 16   (tinyllm section 2.2)
    excess-8:         u - 8                    (ftts int4, "Packing")
    """
    u = np.asarray(u, dtype=np.int64)
    if np.any((u < 0) | (u > 15)):
        raise ValueError("a nibble holds 0..15")
    if enc == TWOS:
        return np.where(u < 8, u, u - 16)
    if enc == EXCESS8:
        return u - 8
    raise ValueError(f"unknown encoding {enc!r}")


def code_to_nibble(q, enc: str) -> np.ndarray:
    """Inverse of nibble_to_code for codes in [-8, 7]."""
    q = np.asarray(q, dtype=np.int64)
    if np.any((q < -8) | (q > 7)):
        raise ValueError("an int4 code lies in [-8, 7]")
    if enc == TWOS:
        return np.where(q >= 0, q, q + 16)
    if enc == EXCESS8:
        return q + 8
    raise ValueError(f"unknown encoding {enc!r}")


def packed_row_bytes(K: int) -> int:
    """Bytes per packed row: two codes per byte, an odd K rounds up."""
    return (K + 1) // 2


def pad_nibble(enc: str) -> int:
    """The stored value that decodes to 0, used for the odd-K pad nibble."""
    return 8 if enc == EXCESS8 else 0


def pack_codes(codes, enc: str) -> np.ndarray:
    """Pack int codes [N, K] into uint8 [N, ceil(K/2)], low nibble = even column."""
    codes = np.asarray(codes, dtype=np.int64)
    if codes.ndim != 2:
        raise ValueError("codes must be [N, K]")
    N, K = codes.shape
    u = code_to_nibble(codes, enc)
    if K % 2:
        u = np.concatenate([u, np.full((N, 1), pad_nibble(enc), np.int64)], axis=1)
    lo = u[:, 0::2]
    hi = u[:, 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_codes(packed, K: int, enc: str) -> np.ndarray:
    """Unpack uint8 [N, ceil(K/2)] into int codes [N, K] (int64)."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.ndim != 2 or packed.shape[1] != packed_row_bytes(K):
        raise ValueError("packed must be [N, ceil(K/2)]")
    b = packed.astype(np.int64)
    lo = b & 0xF          # column 2b
    hi = b >> 4           # column 2b + 1
    u = np.empty((packed.shape[0], 2 * packed.shape[1]), np.int64)
    u[:, 0::2] = lo
    u[:, 1::2] = hi
    return nibble_to_code(u[:, :K], enc)


def unpack_nibbles(packed, K: int) -> np.ndarray:
    """Unpack uint8 [N, ceil(K/2)] into the raw stored nibbles u [N, K] (0..15)."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.ndim != 2 or packed.shape[1] != packed_row_bytes(K):
        raise ValueError("packed must be [N, ceil(K/2)]")
    b = packed.astype(np.int64)
    u = np.empty((packed.shape[0], 2 * packed.shape[1]), np.int64)
    u[:, 0::2] = b & 0xF
    u[:, 1::2] = b >> 4
    return u[:, :K]


def f16_bits_to_float(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 values (subnormals kept).

    numpy's float16 type is the IEEE half format; the conversion to float64
    is exact.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return b.view(np.float16).astype(np.float64)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32: the 16 bits become the top half."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(y) -> np.ndarray:
    """Round finite float32 values to bf16, nearest, ties to even.

    Written from the definition: the two bf16 neighbours of y are its
    truncation and the next bf16 value away from zero; pick the nearer one
    (differences are exact in float64), and on a tie the one whose last
    kept mantissa bit is 0.
    """
    y = np.asarray(y, dtype=np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("finite values only")
    bits = y.view(np.uint32)
    down = (bits & np.uint32(0xFFFF0000))          # toward zero
    up = down + np.uint32(0x10000)                  # away from zero
    v = y.astype(np.float64)
    vd = down.view(np.float32).astype(np.float64)
    vu = up.view(np.float32).astype(np.float64)
    # past the largest finite value the next step up is 2**128 (overflow)
    vu = np.where(np.isinf(vu), np.copysign(2.0 ** 128, v), vu)
    dd = np.abs(v - vd)
    du = np.abs(vu - v)
    even_down = ((down >> np.uint32(16)) & np.uint32(1)) == 0
    take_up = (du < dd) | ((du == dd) & ~even_down)
    out = np.where(take_up, up, down) >> np.uint32(16)
    return out.astype(np.uint16)
