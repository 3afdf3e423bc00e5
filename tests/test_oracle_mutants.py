"""Mutation tests of the oracle's pins (CPU only).

The pitfalls table of "Fused int4 and int8 dequantize-matmul in C" (section 5)
lists twelve plausible bugs, each with the test that catches it.  Each one
that applies to a plain CPU definition is planted here into a copy of the
oracle (through monkeypatch, on the CPU) and at least one pin must fail.
The remaining two concern the C interface and threading and are covered by
the ABI tests (NULL weights -> EINVAL) and the GPU launch-shape tests.
Further mutants cover the quantizer contract (row and matrix), the bf16
rounding, the fixed f32 order of the integer-path epilogues, the per-group
zero points and the condition scale that judges the float paths.
"""
import numpy as np
import pytest

import oracle.formats as F
import oracle.linear as L
import oracle.quantize as Q
from tests import oracle_pins as P

_orig_unpack = F.unpack_codes
_orig_decode = F.nibble_to_code


def _unsigned_decode(u, enc):             # s01: nibbles read as unsigned
    u = np.asarray(u, np.int64)
    return u if enc == F.TWOS else u - 8


def _swapped_unpack(packed, K, enc):      # s02: high nibble taken as the even column
    b = np.asarray(packed, np.int64)
    u = np.empty((b.shape[0], 2 * b.shape[1]), np.int64)
    u[:, 0::2] = b >> 4
    u[:, 1::2] = b & 0xF
    return F.nibble_to_code(u[:, :K], enc)


def _grouped_row0_scales(xf64, codes, scales64, G):   # s03
    return _orig_grouped(xf64, codes, np.broadcast_to(scales64[:1], scales64.shape), G)


def _grouped_no_reset(xf64, codes, scales64, G):      # s04
    M, K = xf64.shape
    y = np.zeros((M, codes.shape[0]))
    partial = np.zeros_like(y)
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        partial = partial + xf64[:, ks] @ codes[:, ks].astype(np.float64).T
        y += partial * scales64[None, :, g]
    return y


def _f16_as_bf16(bits):                               # s05
    return F.bf16_bits_to_f32(bits).astype(np.float64)


def _grouped_first_chunk(xf64, codes, scales64, G):   # s06
    M, K = xf64.shape
    y = np.zeros((M, codes.shape[0]))
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        y += (xf64[:, ks] @ codes[:, :G].astype(np.float64).T) * scales64[None, :, g]
    return y


def _epi_scale_by_m(acc, sx, sw):                     # s07
    a = np.asarray(acc).astype(np.float32)
    M = a.shape[0]
    sw = np.asarray(sw, np.float32)
    t = (a * np.asarray(sx, np.float32)[:, None]).astype(np.float32)
    return (t * sw[np.arange(M) % sw.size][:, None]).astype(np.float32)


def _epi_no_weight_scale(acc, sx, sw):                # s08
    a = np.asarray(acc).astype(np.float32)
    return (a * np.asarray(sx, np.float32)[:, None]).astype(np.float32)


def _epi_grouped_m1_reversed(acc_g, sx, sg):          # s09
    if np.asarray(acc_g).shape[0] != 1:
        return _orig_epi_grouped(acc_g, sx, sg)
    return _orig_epi_grouped(np.asarray(acc_g)[:, :, ::-1], sx, np.asarray(sg)[:, ::-1])


def _no_shape_check(K, G):                            # s10
    return None


def _round_half_away(ratio_like):                     # q1
    r = np.asarray(ratio_like)
    return np.sign(r) * np.floor(np.abs(r) + 0.5)


def _scale_full_range(w, qmax):                       # q2: uses qmax+1 levels
    return _orig_sym(w, qmax + 1)


def _reciprocal(w, qmax):                             # q3: multiply by 1/scale
    w = np.asarray(w, np.float32)
    amax = np.float32(np.max(np.abs(w))) if w.size else np.float32(0)
    scale = np.float32(amax / np.float32(qmax))
    if scale == 0:
        return np.zeros(w.shape, np.int64), np.float32(0)
    inv = np.float32(np.float32(1) / scale)
    q = np.clip(np.rint((w * inv).astype(np.float32)), -qmax, qmax).astype(np.int64)
    return q, scale


def _bf16_truncate(y):                                # b1
    return (np.asarray(y, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _epi_grouped_fused(acc_g, sx, sg):                # e1: one rounding per step
    acc_g = np.asarray(acc_g)
    sg = np.asarray(sg, np.float32)
    t = np.zeros(acc_g.shape[:2], np.float32)
    for g in range(acc_g.shape[2]):
        t = (t.astype(np.float64) + acc_g[:, :, g] * sg[None, :, g].astype(np.float64)).astype(np.float32)
    return (t * np.asarray(sx, np.float32)[:, None]).astype(np.float32)


def _epi_swapped_order(acc, sx, sw):                  # e2: (acc * s_w) * s_x
    a = np.asarray(acc).astype(np.float32)
    t = (a * np.asarray(sw, np.float32)[None, :]).astype(np.float32)
    return (t * np.asarray(sx, np.float32)[:, None]).astype(np.float32)


def _pack_zero_pad(codes, enc):                       # pad: raw 0 as the odd-K pad
    codes = np.asarray(codes, np.int64)
    N, K = codes.shape
    u = F.code_to_nibble(codes, enc)
    if K % 2:
        u = np.concatenate([u, np.zeros((N, 1), np.int64)], axis=1)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def _zp_sign_flipped(qweight, zeros, K, G):          # z1: z - u
    return -_orig_zp_codes(qweight, zeros, K, G)


def _zp_group_by_column(qweight, zeros, K, G):        # z2: z[n, k % Gn]
    u = F.unpack_nibbles(qweight, K)
    z = np.asarray(zeros, np.int64).reshape(u.shape[0], K // G)
    return u - np.tile(z, (1, G))


def _zp_ignored(qweight, zeros, K, G):                 # z3: the constant 8 kept
    return F.unpack_nibbles(qweight, K) - 8


def _per_row_scale_by_m(xf64, wq, sw):                # w1: per-row scale indexed by the activation row
    q = np.asarray(wq, np.int8).astype(np.float64)
    s = np.asarray(sw, np.float32).astype(np.float64).reshape(-1)
    M = xf64.shape[0]
    return (xf64 @ q.T) * s[np.arange(M) % s.size][:, None]


def _per_row_unsigned(xf64, wq, sw):                  # w2: int8 codes read as unsigned bytes
    q = np.asarray(wq, np.int8).view(np.uint8).astype(np.float64)
    return (xf64 @ q.T) * np.asarray(sw, np.float32).astype(np.float64).reshape(-1)[None, :]


def _abs_terms_signed_codes(x64, qweight, scales64, K, G, enc):   # c1: |q| forgotten
    codes = L.unpack_codes(qweight, K, enc).astype(np.float64)
    return L._grouped_float(np.abs(np.asarray(x64, np.float64)), codes, np.abs(np.asarray(scales64, np.float64)), G)


def _abs_terms_signed_x(x64, qweight, scales64, K, G, enc):       # c2: |x| forgotten
    codes = np.abs(L.unpack_codes(qweight, K, enc)).astype(np.float64)
    return L._grouped_float(np.asarray(x64, np.float64), codes, np.abs(np.asarray(scales64, np.float64)), G)


def _abs_terms_signed_scales(x64, qweight, scales64, K, G, enc):  # c3: |s| forgotten
    codes = np.abs(L.unpack_codes(qweight, K, enc)).astype(np.float64)
    return L._grouped_float(np.abs(np.asarray(x64, np.float64)), codes, np.asarray(scales64, np.float64), G)


def _abs_of_sum(x64, qweight, scales64, K, G, enc):               # c4: |sum| instead of sum of |terms|
    codes = L.unpack_codes(qweight, K, enc).astype(np.float64)
    return np.abs(L._grouped_float(np.asarray(x64, np.float64), codes, np.asarray(scales64, np.float64), G))


def _matrix_global_scale(W):                                     # m1: one scale for the whole matrix
    W = np.asarray(W, dtype=np.float32)
    K = W.shape[1]
    if W.shape[0] == 0:
        return np.zeros((0, (K + 1) // 2), np.uint8), np.zeros(0, np.float32)
    s = np.float32(np.float32(np.abs(W).max()) / np.float32(7))
    q = np.zeros(W.shape, np.int64) if s == 0 else np.clip(np.rint((W / s).astype(np.float32)), -7, 7).astype(np.int64)
    return F.pack_codes(q, F.EXCESS8), np.full(W.shape[0], s, np.float32)


def _matrix_scales_shifted(W):                                   # m2: scales stored one row off
    p, s = _orig_q4_matrix(W)
    return p, np.roll(s, 1)


_orig_q4_matrix = Q.quantize_q4_matrix
_orig_grouped = L._grouped_float
_orig_epi_grouped = L.epilogue_grouped
_orig_sym = Q._symmetric_row
_orig_zp_codes = L.codes_with_zero_points

MUTANTS = {
    "s01_unsigned_nibbles": [(F, "nibble_to_code", _unsigned_decode)],
    "s02_high_nibble_even_column": [(F, "unpack_codes", _swapped_unpack), (L, "unpack_codes", _swapped_unpack)],
    "s03_scales_by_group_only": [(L, "_grouped_float", _grouped_row0_scales)],
    "s04_partial_not_reset": [(L, "_grouped_float", _grouped_no_reset)],
    "s05_f16_read_as_bf16": [(F, "f16_bits_to_float", _f16_as_bf16), (L, "f16_bits_to_float", _f16_as_bf16)],
    "s06_first_group_codes": [(L, "_grouped_float", _grouped_first_chunk)],
    "s07_int8_scale_by_row_m": [(L, "epilogue_per_channel", _epi_scale_by_m)],
    "s08_int8_scale_forgotten": [(L, "epilogue_per_channel", _epi_no_weight_scale)],
    "s09_special_order_m1": [(L, "epilogue_grouped", _epi_grouped_m1_reversed)],
    "s10_group_not_dividing_k": [(L, "check_group_shape", _no_shape_check)],
    "q1_round_half_away": [(np, "rint", _round_half_away)],
    "q2_min_code_emitted": [(Q, "_symmetric_row", _scale_full_range)],
    "q3_reciprocal_multiply": [(Q, "_symmetric_row", _reciprocal)],
    "b1_bf16_truncation": [(F, "f32_to_bf16_bits", _bf16_truncate)],
    "e1_grouped_single_rounding": [(L, "epilogue_grouped", _epi_grouped_fused)],
    "e2_scale_order_swapped": [(L, "epilogue_per_channel", _epi_swapped_order)],
    "pad_raw_zero": [(F, "pack_codes", _pack_zero_pad), (Q, "pack_codes", _pack_zero_pad)],
    "z1_zero_point_sign": [(L, "codes_with_zero_points", _zp_sign_flipped)],
    "z2_zero_point_group_by_column": [(L, "codes_with_zero_points", _zp_group_by_column)],
    "z3_zero_point_ignored": [(L, "codes_with_zero_points", _zp_ignored)],
    "w1_int8_row_scale_by_m": [(L, "_per_row_float", _per_row_scale_by_m)],
    "w2_int8_codes_unsigned": [(L, "_per_row_float", _per_row_unsigned)],
    "c1_abs_terms_signed_codes": [(L, "abs_terms", _abs_terms_signed_codes)],
    "c2_abs_terms_signed_x": [(L, "abs_terms", _abs_terms_signed_x)],
    "c3_abs_terms_signed_scales": [(L, "abs_terms", _abs_terms_signed_scales)],
    "c4_abs_terms_abs_of_sum": [(L, "abs_terms", _abs_of_sum)],
    "m1_matrix_global_scale": [(Q, "quantize_q4_matrix", _matrix_global_scale)],
    "m2_matrix_scales_shifted": [(Q, "quantize_q4_matrix", _matrix_scales_shifted)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTANTS[name]:
        monkeypatch.setattr(mod, attr, fn)
    failed = P.run_all(seed=3)
    assert failed, f"mutant {name} survived every pin"


def test_unmutated_oracle_passes_every_pin():
    assert P.run_all(seed=3) == []
