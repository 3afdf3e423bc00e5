"""Pins of the oracle: checks against what the pages and mathematics fix.

Each check_* function raises AssertionError when the oracle is wrong.  They
are called by test_oracle_pins.py on the oracle as written and by
test_oracle_mutants.py on deliberately broken copies (each plausible mistake
must fail at least one check).  Function lookups go through the module
objects at call time so a patched function is the one exercised.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

import oracle.errors as E
import oracle.formats as F
import oracle.linear as L
import oracle.quantize as Q
from tests import exact_ref as X

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _hex(s):
    return int(s, 16)


# --------------------------------------------------------------------------
# worked example (tinyllm section 3) on every linear
# --------------------------------------------------------------------------

def check_hand_example_w4a32():
    g = _golden("worked_example.json")
    codes = np.array(g["codes"])
    packed = F.pack_codes(codes, F.TWOS)
    assert packed.tolist() == [[_hex(b) for b in r] for r in g["bytes"]], packed
    scales = np.array([[_hex(b) for b in r] for r in g["scales_f16_bits"]], np.uint16)
    x = np.array([g["x"]], np.float32)
    y = L.linear_w4a32(x, packed, scales, g["G"], F.TWOS)
    assert y.tolist() == [g["y"]], y


def check_q8_hand_example():
    """int8 weights with the same codes and one scale per row -> [-13, 5]."""
    g = _golden("worked_example.json")
    wq = np.array(g["codes"], np.int8)
    xq = np.array([g["x"]], np.int8)
    y = L.linear_w8a8(xq, np.array([1.0], np.float32), wq, np.array(g["int8_row_scales"], np.float32))
    assert y.tolist() == [g["int8_y"]], y


def check_q8_hand_example_float_activations():
    """The int8 variant of the worked example with float activations (f32 and
    bf16: 1, 2, 3, 4 are exact in both) -> [-13, 5], exactly."""
    g = _golden("worked_example.json")
    wq = np.array(g["codes"], np.int8)
    sw = np.array(g["int8_row_scales"], np.float32)
    x = np.array([g["x"]], np.float32)
    assert L.linear_w8a32(x, wq, sw).tolist() == [g["int8_y"]]
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert L.linear_w8a16(xb, wq, sw).tolist() == [g["int8_y"]]


def check_w8_float_exact(rng):
    """W8A32 / W8A16 against exact rationals on random rows (int8 codes over
    the full range, including -128), and W8A32 with codes in [-8, 7] against
    the W4A32 oracle with one group per row (same factored sum)."""
    M, N, K = 2, 3, 40
    wq = rng.integers(-128, 128, (N, K)).astype(np.int8)
    sw = rng.uniform(0.001, 0.05, N).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    y32, y16 = L.linear_w8a32(x, wq, sw), L.linear_w8a16(xb, wq, sw)
    for m in range(M):
        for n in range(N):
            sv = X.f32_value(int(sw.view(np.uint32)[n]))
            for y, xv in ((y32, [X.f32_value(int(b)) for b in x[m].view(np.uint32)]),
                          (y16, [X.bf16_value(int(b)) for b in xb[m]])):
                terms = [xv[k] * int(wq[n, k]) * sv for k in range(K)]
                bound = K * Fraction(2) ** -52 * sum(abs(t) for t in terms)
                assert abs(Fraction(float(y[m, n])) - sum(terms, Fraction(0))) <= bound, (m, n)
    codes = rng.integers(-8, 8, (N, K))
    s16 = np.array(rng.uniform(0.001, 0.05, N), np.float16)
    y8 = L.linear_w8a32(x, codes.astype(np.int8), s16.astype(np.float32))
    y4 = L.linear_w4a32(x, F.pack_codes(codes, F.TWOS), s16.view(np.uint16).reshape(N, 1), K, F.TWOS)
    assert np.allclose(y8, y4, rtol=0, atol=4 * K * 2.0 ** -52 * np.abs(y4).max())


def check_hand_example_w4a8():
    """The same example through the W4A8 forms (per channel and grouped)."""
    g = _golden("worked_example.json")
    codes = np.array(g["codes"])
    packed8 = F.pack_codes(codes, F.EXCESS8)
    # stored value = code + 8: row 0 -> 9,6,11,0 ; row 1 -> 15,8,7,12
    assert packed8.tolist() == [[0x69, 0x0B], [0x8F, 0xC7]], packed8
    xq = np.array([g["x"]], np.int8)
    one = np.array([1.0], np.float32)
    y = L.linear_w4a8(xq, one, packed8, np.array(g["int8_row_scales"], np.float32), 0, F.EXCESS8)
    assert y.tolist() == [g["int8_y"]], y
    y = L.linear_w4a8(xq, one, packed8, np.array(g["scale_values"], np.float32), g["G"], F.EXCESS8)
    assert y.tolist() == [g["y"]], y
    # two's-complement storage of the same codes gives the same results
    packed2 = F.pack_codes(codes, F.TWOS)
    y = L.linear_w4a8(xq, one, packed2, np.array(g["scale_values"], np.float32), g["G"], F.TWOS)
    assert y.tolist() == [g["y"]], y


def check_hand_example_w4a16():
    g = _golden("worked_example.json")
    codes = np.array(g["codes"])
    # bf16 patterns of 1, 2, 3, 4 and of the scales 0.5, 2, 1, 0.25
    x_bits = np.array([[0x3F80, 0x4000, 0x4040, 0x4080]], np.uint16)
    s_bits = np.array([[0x3F00, 0x4000], [0x3F80, 0x3E80]], np.uint16)
    for enc in F.ENCODINGS:
        y = L.linear_w4a16(x_bits, F.pack_codes(codes, enc), s_bits, g["G"], enc)
        assert y.tolist() == [g["y"]], (enc, y)


# --------------------------------------------------------------------------
# formats
# --------------------------------------------------------------------------

def check_every_nibble_code():
    g = _golden("nibble_codes.json")
    for enc in F.ENCODINGS:
        for u in range(16):
            # u in the low nibble next to a fixed high nibble, then the reverse
            lo_byte = np.array([[u | (0x3 << 4)]], np.uint8)
            hi_byte = np.array([[0x5 | (u << 4)]], np.uint8)
            c_lo = F.unpack_codes(lo_byte, 2, enc)[0]
            c_hi = F.unpack_codes(hi_byte, 2, enc)[0]
            assert c_lo[0] == g[enc][u], (enc, u, c_lo)
            assert c_lo[1] == g[enc][3], (enc, u, c_lo)
            assert c_hi[1] == g[enc][u], (enc, u, c_hi)
            assert c_hi[0] == g[enc][5], (enc, u, c_hi)


def check_f16_scales_decode_exactly():
    g = _golden("f16_scales.json")
    for case in g["cases"]:
        bits = _hex(case["bits"])
        got = F.f16_bits_to_float(np.array([bits], np.uint16))[0]
        want = X.f16_value(bits)
        assert Fraction(got) == want, (case, got)
        if case["value"] is not None:
            assert got == case["value"]
    # every finite pattern against the IEEE binary16 definition
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = F.f16_bits_to_float(allbits)
    for b in range(0, 1 << 16, 7):
        want = X.f16_value(b)
        if want is not None:
            assert Fraction(vals[b]) == want, hex(b)


def check_bf16_decode():
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_bits_to_f32(allbits)
    for b in range(0, 1 << 16, 5):
        want = X.bf16_value(b)
        if want is not None:
            assert Fraction(float(vals[b])) == want, hex(b)


def check_bf16_rounding(rng):
    # hand ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> 1 (even);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6 (even)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0], np.float32)
    assert F.f32_to_bf16_bits(ties).tolist() == [0x3F80, 0x3F82, 0xBF80, 0x0000]
    v = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32)
    v = np.concatenate([v, np.array([np.finfo(np.float32).max, 1e-40, -3e-39], np.float32)])
    got = F.f32_to_bf16_bits(v)
    for i in range(v.size):
        want = X.round_to_bf16(X.f32_value(int(v.view(np.uint32)[i])))
        gv = X.bf16_value(int(got[i]))
        if gv is None:   # rounded past the largest finite bf16
            assert abs(want) >= X.bf16_value(0x7F7F), (v[i], got[i])
        else:
            assert gv == want, (v[i], hex(int(got[i])))


def check_pack_roundtrip():
    for enc in F.ENCODINGS:
        lo_hi = [(a, b) for a in range(-8, 8) for b in range(-8, 8)]
        codes = np.array([[a, b] for a, b in lo_hi])
        packed = F.pack_codes(codes, enc)
        assert np.array_equal(F.unpack_codes(packed, 2, enc), codes)
        # the byte holds the even column in bits 0-3
        for (a, b), byte in zip(lo_hi, packed[:, 0]):
            assert X.decode_nibble_rule(int(byte) & 0xF, enc) == a
            assert X.decode_nibble_rule(int(byte) >> 4, enc) == b
        # long rows at every position, odd and even K
        rng = np.random.default_rng(7)
        for K in (1, 2, 3, 31, 64, 1023):
            codes = rng.integers(-8, 8, (5, K))
            packed = F.pack_codes(codes, enc)
            assert packed.shape == (5, (K + 1) // 2)
            assert np.array_equal(F.unpack_codes(packed, K, enc), codes)
            assert X.unpack_byte_rows(packed, K, enc) == codes.tolist()


def check_odd_k_pad():
    codes = np.array([[1, -2, 3]])
    p = F.pack_codes(codes, F.EXCESS8)
    assert p.shape == (1, 2)
    assert (int(p[0, 1]) >> 4) == 8          # the biased zero, not a raw 0
    assert X.decode_nibble_rule(8, "excess8") == 0
    # whole-byte reading (K rounded up) gives the same W4A8 result as K
    xq = np.array([[5, -7, 9, 100]], np.int8)
    sw = np.array([0.5], np.float32)
    sx = np.array([0.25], np.float32)
    y_k = L.linear_w4a8(xq[:, :3], sx, p, sw, 0, F.EXCESS8)
    y_whole = L.linear_w4a8(xq, sx, p, sw, 0, F.EXCESS8)
    assert np.array_equal(y_k, y_whole)


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def check_quantizer_ties():
    w = np.array([7, .5, 1.5, 2.5, -.5, -1.5, -2.5], np.float32)
    packed, s = Q.quantize_q4_row(w)
    assert s == np.float32(1.0)
    assert F.unpack_codes(packed[None], 7, F.EXCESS8)[0].tolist() == [7, 0, 2, 2, 0, -2, -2]
    assert packed.tolist() == [0x8F, 0xAA, 0x68, 0x86]
    q8, s8 = Q.quantize_q8_row(np.array([127, .5, 1.5, 2.5, -.5, -1.5, -2.5], np.float32))
    assert s8 == np.float32(1.0)
    assert q8.tolist() == [127, 0, 2, 2, 0, -2, -2]
    # the quotient, not a product with a rounded reciprocal: scale 7 exactly,
    # 45.5 / 7 = 6.5 is a tie (-> 6) while 45.5 * fl(1/7) rounds to 7
    q4c, s4 = Q.quantize_q4_codes_row(np.array([49, 45.5, -45.5], np.float32))
    assert s4 == np.float32(7.0) and q4c.tolist() == [7, 6, -6]
    q8c, s8c = Q.quantize_q8_row(np.array([889, 45.5, -45.5], np.float32))
    assert s8c == np.float32(7.0) and q8c.tolist() == [127, 6, -6]
    # all-zero row: scale 0, codes 0 (stored as the biased zero)
    p0, s0 = Q.quantize_q4_row(np.zeros(5, np.float32))
    assert s0 == 0 and p0.tolist() == [0x88, 0x88, 0x88]


def check_quantize_matrix():
    """The matrix quantizer row by row on hand-derived rows (golden
    quantizer_matrix.json): the tie row, its negation, a zero row, the row
    doubled and a single value, at odd K; each row's own scale and bytes,
    in row order, and the same as the one-row quantizer."""
    g = _golden("quantizer_matrix.json")
    W = np.array(g["rows"], np.float32)
    packed, scales = Q.quantize_q4_matrix(W)
    assert packed.shape == (W.shape[0], (g["K"] + 1) // 2), packed.shape
    assert scales.dtype == np.float32 and scales.tolist() == g["scales"], scales
    assert packed.tolist() == [[_hex(b) for b in r] for r in g["bytes"]], packed
    assert F.unpack_codes(packed, g["K"], F.EXCESS8).tolist() == g["codes"]
    for n in range(W.shape[0]):
        p1, s1 = Q.quantize_q4_row(W[n])
        assert p1.tolist() == packed[n].tolist() and s1 == scales[n], n
    # an empty matrix keeps its row width
    p0, s0 = Q.quantize_q4_matrix(np.zeros((0, 7), np.float32))
    assert p0.shape == (0, 4) and s0.shape == (0,)


def check_abs_terms_closed_form():
    """sum_k |x q s| on rows whose every term has the same magnitude:
    |x| = 1.5, |q| = 8 (code -8 in both encodings), |s| = 0.25 with mixed
    signs everywhere, so c = 3 K exactly for every output."""
    K, G = 12, 4
    for enc in F.ENCODINGS:
        codes = np.full((3, K), -8)
        packed = F.pack_codes(codes, enc)
        x = np.array([[1.5, -1.5] * (K // 2), [-1.5] * K], np.float64)
        s = np.array([[0.25, -0.25, 0.25], [-0.25] * 3, [0.25] * 3], np.float64)
        c = L.abs_terms(x, packed, s, K, G, enc)
        assert c.tolist() == [[3.0 * K] * 3] * 2, (enc, c)


def check_abs_terms_exact(rng):
    """The condition scale c[m,n] = sum_k |x[m,k] q[n,k] s[n,k//G]| against
    exact rationals from a literal byte-by-byte unpack: random signs in x,
    in the codes and in the scales, every group size of K = 12; c is a sum
    of non-negative float64 terms, so it lies within K 2^-52 c of the exact
    value."""
    K = 12
    for G in (2, 4, 6, 12):
        for enc in F.ENCODINGS:
            M, N = 2, 3
            codes, packed = _random_w4(rng, N, K, G, enc)
            s = rng.uniform(-0.03, 0.03, (N, K // G)).astype(np.float32).astype(np.float64)
            x = rng.standard_normal((M, K)).astype(np.float32)
            c = L.abs_terms(x.astype(np.float64), packed, s, K, G, enc)
            assert c.shape == (M, N)
            cols = X.unpack_byte_rows(packed, K, enc)
            xv = [[X.f32_value(int(b)) for b in row] for row in x.view(np.uint32)]
            sv = [[Fraction(float(v)) for v in row] for row in s]
            for m in range(M):
                for n in range(N):
                    exact = sum((abs(xv[m][k] * cols[n][k] * sv[n][k // G]) for k in range(K)), Fraction(0))
                    assert abs(Fraction(float(c[m, n])) - exact) <= K * Fraction(2) ** -52 * exact, (G, enc, m, n)


def check_quantizer_exact(rng):
    """Codes and scale equal the exact-rational statement of the recipe."""
    for qmax, fn in ((7, Q.quantize_q4_codes_row), (127, Q.quantize_q8_row)):
        for _ in range(20):
            K = int(rng.integers(1, 40))
            w = (rng.standard_normal(K) * 0.02).astype(np.float32)
            q, s = fn(w)
            wv = [X.f32_value(int(b)) for b in w.view(np.uint32)]
            amax = max(abs(v) for v in wv)
            s_ref = X.round_to_binary32(amax / qmax)
            assert Fraction(float(s)) == s_ref
            for v, qi in zip(wv, np.asarray(q).tolist()):
                r = X.round_to_binary32(v / s_ref)
                fl = r.numerator // r.denominator
                rem = r - fl
                want = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
                want = max(-qmax, min(qmax, want))
                assert qi == want, (v, qi, want)


def check_no_min_code(rng):
    for _ in range(200):
        K = int(rng.integers(1, 64))
        w = (rng.standard_normal(K) * np.exp2(rng.integers(-20, 20))).astype(np.float32)
        if rng.integers(0, 2):
            w[rng.integers(0, K)] = -np.abs(w).max() * 1.0   # a row whose minimum is the extreme
        q, _ = Q.quantize_q4_codes_row(w)
        assert q.min() >= -7 and q.max() <= 7
        q8, _ = Q.quantize_q8_row(w)
        assert q8.min() >= -127 and q8.max() <= 127


def check_negation(rng):
    for _ in range(100):
        K = int(rng.integers(1, 64))
        w = (rng.standard_normal(K) * 0.02).astype(np.float32)
        q, s = Q.quantize_q4_codes_row(w)
        qn, sn = Q.quantize_q4_codes_row(-w)
        assert s == sn and np.array_equal(qn, -q)
        q8, s8 = Q.quantize_q8_row(w)
        q8n, s8n = Q.quantize_q8_row(-w)
        assert s8 == s8n and np.array_equal(q8n, -q8)


# --------------------------------------------------------------------------
# linears against closed forms and exact brute force
# --------------------------------------------------------------------------

def check_all_extreme():
    """xq = +-127 against q = +-7 (or -8 when grouped): acc = +-889 K (+-1016 K)."""
    for K in (64, 5632):
        xq = np.full((2, K), 127, np.int8)
        xq[1] = -127
        codes = np.full((2, K), 7)
        codes[1] = -7
        packed = F.pack_codes(codes, F.EXCESS8)
        one = np.ones(2, np.float32)
        y = L.linear_w4a8(xq, one, packed, one, 0, F.EXCESS8)
        assert y.tolist() == [[889.0 * K, -889.0 * K], [-889.0 * K, 889.0 * K]], y
        codes8 = np.full((1, K), -8)
        packed8 = F.pack_codes(codes8, F.TWOS)
        y = L.linear_w4a8(xq[:1], one[:1], packed8, np.ones((1, K // 64), np.float32), 64, F.TWOS)
        assert y.tolist() == [[-1016.0 * K]], y


def check_index_probe():
    """Codes that name their own position, read back through one-hot x."""
    N, K, G = 6, 16, 4
    codes = ((np.arange(N)[:, None] * 3 + np.arange(K)[None, :] * 5) % 16) - 8
    for enc in F.ENCODINGS:
        packed = F.pack_codes(codes, enc)
        ones = np.full((N, K // G), 0x3C00, np.uint16)          # f16 1.0
        x = np.eye(K, dtype=np.float32)                          # row m picks column m
        y = L.linear_w4a32(x, packed, ones, G, enc)
        assert np.array_equal(y, codes.T.astype(np.float64)), enc
        xq = np.eye(K, dtype=np.int8)
        y8 = L.linear_w4a8(xq, np.ones(K, np.float32), packed, np.ones(N, np.float32), 0, enc)
        assert np.array_equal(y8, codes.T.astype(np.float32)), enc


def _random_w4(rng, N, K, G, enc):
    codes = rng.integers(-8, 8, (N, K))
    return codes, F.pack_codes(codes, enc)


def check_matches_dequantize_then_matmul(rng):
    """The fused factorised sum equals the obvious recipe (float64 and exact)."""
    K = 384
    for G in (2, 32, 64, K):
        for enc in F.ENCODINGS:
            M, N = 3, 37
            codes, packed = _random_w4(rng, N, K, G, enc)
            s_bits = np.array(rng.uniform(0.001, 0.02, (N, K // G)), np.float16).view(np.uint16)
            x = rng.standard_normal((M, K)).astype(np.float32)
            y = L.linear_w4a32(x, packed, s_bits, G, enc)
            W = L.dequantize_w4(packed, F.f16_bits_to_float(s_bits), K, G, enc)
            y_ref = x.astype(np.float64) @ W.T
            c = np.abs(x.astype(np.float64)) @ np.abs(W).T
            assert np.all(np.abs(y - y_ref) <= 2 * K * 2.0 ** -52 * c), (G, enc)
    # exact rationals on a tiny case, every group size that divides K
    K = 12
    for G in (2, 4, 6, 12):
        M, N = 2, 3
        enc = F.TWOS
        codes, packed = _random_w4(rng, N, K, G, enc)
        s_bits = np.array(rng.uniform(0.001, 0.02, (N, K // G)), np.float16).view(np.uint16)
        x = rng.standard_normal((M, K)).astype(np.float32)
        y = L.linear_w4a32(x, packed, s_bits, G, enc)
        cols = X.unpack_byte_rows(packed, K, enc)
        wv = [[cols[n][k] * X.f16_value(int(s_bits[n, k // G])) for k in range(K)] for n in range(N)]
        xv = [[X.f32_value(int(b)) for b in row] for row in x.view(np.uint32)]
        ye = X.exact_matmul_dequant(xv, wv)
        for m in range(M):
            for n in range(N):
                bound = K * Fraction(2) ** -52 * sum(abs(a * b) for a, b in zip(xv[m], wv[n]))
                assert abs(Fraction(float(y[m, n])) - ye[m][n]) <= bound, (G, m, n)


def check_q8_matches_dequantize_then_matmul(rng):
    """W8A8 / W4A8 per channel at K = 200 and M > 1 against exact replay."""
    M, N, K = 3, 5, 200
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sx = rng.uniform(0.001, 0.1, M).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, N).astype(np.float32)
    y = L.linear_w8a8(xq, sx, wq, sw)
    codes = rng.integers(-7, 8, (N, K))
    y4 = L.linear_w4a8(xq, sx, F.pack_codes(codes, F.EXCESS8), sw, 0, F.EXCESS8)
    for m in range(M):
        for n in range(N):
            for out, wrow in ((y, wq[n].tolist()), (y4, codes[n].tolist())):
                acc = sum(int(a) * int(b) for a, b in zip(xq[m].tolist(), wrow))
                t = X.round_to_binary32(X.round_to_binary32(Fraction(acc)) * X.f32_value(int(sx.view(np.uint32)[m])))
                want = X.round_to_binary32(t * X.f32_value(int(sw.view(np.uint32)[n])))
                assert Fraction(float(out[m, n])) == want, (m, n)


def check_grouped_w4a8_exact(rng):
    """Grouped W4A8: the f32 sequence over groups replayed in exact rationals,
    and the result within the rounding bound of the exact real value."""
    M, N, K, G = 2, 4, 48, 8
    for enc in F.ENCODINGS:
        codes, packed = _random_w4(rng, N, K, G, enc)
        xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
        sx = rng.uniform(0.001, 0.1, M).astype(np.float32)
        sg = rng.uniform(0.002, 0.03, (N, K // G)).astype(np.float32)
        y = L.linear_w4a8(xq, sx, packed, sg, G, enc)
        cols = X.unpack_byte_rows(packed, K, enc)
        for m in range(M):
            sxv = X.f32_value(int(sx.view(np.uint32)[m]))
            for n in range(N):
                accs = [sum(int(xq[m, k]) * cols[n][k] for k in range(g * G, (g + 1) * G))
                        for g in range(K // G)]
                sv = [X.f32_value(int(b)) for b in sg[n].view(np.uint32)]
                t = X.round_to_binary32(X.round_to_binary32(Fraction(accs[0])) * sv[0])
                for g in range(1, K // G):
                    t = X.round_to_binary32(t + X.round_to_binary32(X.round_to_binary32(Fraction(accs[g])) * sv[g]))
                want = X.round_to_binary32(t * sxv)
                assert Fraction(float(y[m, n])) == want, (enc, m, n)
                exact = sxv * sum(a * s for a, s in zip(accs, sv))
                mag = sxv * sum(abs(a * s) for a, s in zip(accs, sv))
                assert abs(want - exact) <= (K // G + 2) * Fraction(2) ** -24 * mag


def check_w4a16_exact(rng):
    M, N, K, G = 2, 3, 16, 8
    for enc in F.ENCODINGS:
        codes, packed = _random_w4(rng, N, K, G, enc)
        xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        sb = (rng.uniform(0.002, 0.03, (N, K // G)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        y = L.linear_w4a16(xb, packed, sb, G, enc)
        cols = X.unpack_byte_rows(packed, K, enc)
        for m in range(M):
            for n in range(N):
                terms = [X.bf16_value(int(xb[m, k])) * cols[n][k] * X.bf16_value(int(sb[n, k // G]))
                         for k in range(K)]
                exact = sum(terms, Fraction(0))
                bound = K * Fraction(2) ** -52 * sum(abs(t) for t in terms)
                assert abs(Fraction(float(y[m, n])) - exact) <= bound


def check_batch_invariant_rows(rng):
    """Integer-activation rows alone vs in a batch: bitwise equal."""
    M, N, K, G = 12, 9, 64, 16
    codes, packed = _random_w4(rng, N, K, G, F.EXCESS8)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = rng.uniform(0.001, 0.1, M).astype(np.float32)
    sg = rng.uniform(0.002, 0.03, (N, K // G)).astype(np.float32)
    yb = L.linear_w4a8(xq, sx, packed, sg, G, F.EXCESS8)
    for m in range(M):
        y1 = L.linear_w4a8(xq[m:m + 1], sx[m:m + 1], packed, sg, G, F.EXCESS8)
        assert np.array_equal(y1[0], yb[m]), m


def check_shape_errors():
    packed = np.zeros((2, 2), np.uint8)
    x = np.zeros((1, 4), np.float32)
    s = np.zeros((2, 2), np.uint16)
    for G in (0, -2, 3, 8):
        try:
            L.linear_w4a32(x, packed, s, G, F.TWOS)
        except ValueError:
            continue
        raise AssertionError(f"group {G} accepted for K=4")


def check_error_measures():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    y = np.array([[1.0, -2.0, 1e-6]])
    assert E.normwise(y, y_ref) == 1e-6 / 2.0
    assert E.conditioned(y, y_ref, np.array([[1.0, 1.0, 4.0]])) == 1e-6 / 4.0
    assert E.normwise(y_ref, y_ref) == 0.0


def check_dynamic_w4a8(rng):
    """Dynamic W4A8 = quantize rows with the Q8 recipe, then the W4A8 linear."""
    M, N, K = 3, 4, 33
    x = rng.standard_normal((M, K)).astype(np.float32)
    codes = rng.integers(-7, 8, (N, K))
    packed = F.pack_codes(codes, F.EXCESS8)
    sw = rng.uniform(0.001, 0.01, N).astype(np.float32)
    y, xq, sx = L.linear_w4a8_dynamic(x, packed, sw, 0, F.EXCESS8, "f32")
    for m in range(M):
        q, s = Q.quantize_q8_row(x[m])
        assert np.array_equal(q, xq[m]) and s == sx[m]
    assert np.array_equal(y, L.linear_w4a8(xq, sx, packed, sw, 0, F.EXCESS8))
    # bf16 activations widen exactly before quantizing
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    _, xqb, sxb = L.linear_w4a8_dynamic(xb, packed, sw, 0, F.EXCESS8, "bf16")
    for m in range(M):
        q, s = Q.quantize_q8_row((xb[m].astype(np.uint32) << 16).view(np.float32))
        assert np.array_equal(q, xqb[m]) and s == sxb[m]


# --------------------------------------------------------------------------
# per-group zero points ("The 4-bit CPU path", section "W4A8")
# --------------------------------------------------------------------------

def _literal_zp_codes(packed, zeros, K, G):
    """q[n][k] = u - z[n][k // G], u read byte by byte (bits 0-3 = column 2b)."""
    rows = []
    for n, row in enumerate(packed):
        us = []
        for b in row:
            us += [int(b) & 0xF, (int(b) >> 4) & 0xF]
        rows.append([us[k] - int(zeros[n][k // G]) for k in range(K)])
    return rows


def check_zero_points_reduce_to_symmetric(rng):
    """A zero point of 8 in every group is the symmetric excess-8 layout."""
    M, N, K, G = 3, 7, 64, 16
    codes, packed = _random_w4(rng, N, K, G, F.EXCESS8)
    z8 = np.full((N, K // G), 8, np.uint8)
    xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sb = (rng.uniform(0.002, 0.03, (N, K // G)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(L.linear_w4a16_zp(xb, packed, sb, z8, G), L.linear_w4a16(xb, packed, sb, G, F.EXCESS8))
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = rng.uniform(0.001, 0.1, M).astype(np.float32)
    sg = rng.uniform(0.002, 0.03, (N, K // G)).astype(np.float32)
    assert np.array_equal(L.linear_w4a8_zp(xq, sx, packed, sg, z8, G).view(np.uint32),
                          L.linear_w4a8(xq, sx, packed, sg, G, F.EXCESS8).view(np.uint32))


def check_zero_points_closed_forms():
    """Stored nibble == zero point everywhere: every weight is 0, y = 0.
    One-hot x at column k reads s[n, k // G] * (u[n,k] - z[n, k // G])."""
    N, K, G = 5, 24, 8
    Gn = K // G
    z = (np.arange(N * Gn).reshape(N, Gn) * 7 + 3) % 16
    u = np.repeat(z, G, axis=1)
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    xb = np.full((2, K), 0x3F80, np.uint16)                                   # x = 1.0
    sb = np.full((N, Gn), 0x3F80, np.uint16)
    assert np.all(L.linear_w4a16_zp(xb, packed, sb, z.astype(np.uint8), G) == 0.0)
    xq = np.full((2, K), 127, np.int8)
    y8 = L.linear_w4a8_zp(xq, np.ones(2, np.float32), packed, np.ones((N, Gn), np.float32),
                          z.astype(np.uint8), G)
    assert np.all(y8 == 0.0)
    u2 = (np.arange(N * K).reshape(N, K) * 5 + 1) % 16
    packed2 = (u2[:, 0::2] | (u2[:, 1::2] << 4)).astype(np.uint8)
    s_vals = np.array([[2.0 ** -(n + g + 1) for g in range(Gn)] for n in range(N)], np.float32)
    sb2 = (s_vals.view(np.uint32) >> 16).astype(np.uint16)
    for k in range(K):
        xk = np.zeros((1, K), np.uint16)
        xk[0, k] = 0x3F80
        y = L.linear_w4a16_zp(xk, packed2, sb2, z.astype(np.uint8), G)[0]
        want = [(int(u2[n, k]) - int(z[n, k // G])) * float(s_vals[n, k // G]) for n in range(N)]
        assert np.array_equal(y, np.array(want)), k


def check_zero_points_exact(rng):
    """Random zero points per group, literal unpack, exact rationals: W4A16
    within the rounding bound, grouped W4A8 replayed bit for bit."""
    M, N, K, G = 2, 4, 48, 8
    Gn = K // G
    u = rng.integers(0, 16, (N, K))
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    zeros = rng.integers(0, 16, (N, Gn)).astype(np.uint8)
    cols = _literal_zp_codes(packed, zeros, K, G)
    xb = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sb = (rng.uniform(0.002, 0.03, (N, Gn)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = L.linear_w4a16_zp(xb, packed, sb, zeros, G)
    for m in range(M):
        for n in range(N):
            terms = [X.bf16_value(int(xb[m, k])) * cols[n][k] * X.bf16_value(int(sb[n, k // G]))
                     for k in range(K)]
            bound = K * Fraction(2) ** -52 * sum(abs(t) for t in terms)
            assert abs(Fraction(float(y[m, n])) - sum(terms, Fraction(0))) <= bound, (m, n)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    sx = rng.uniform(0.001, 0.1, M).astype(np.float32)
    sg = rng.uniform(0.002, 0.03, (N, Gn)).astype(np.float32)
    y8 = L.linear_w4a8_zp(xq, sx, packed, sg, zeros, G)
    for m in range(M):
        sxv = X.f32_value(int(sx.view(np.uint32)[m]))
        for n in range(N):
            accs = [sum(int(xq[m, k]) * cols[n][k] for k in range(g * G, (g + 1) * G)) for g in range(Gn)]
            sv = [X.f32_value(int(b)) for b in sg[n].view(np.uint32)]
            t = X.round_to_binary32(X.round_to_binary32(Fraction(accs[0])) * sv[0])
            for g in range(1, Gn):
                t = X.round_to_binary32(t + X.round_to_binary32(X.round_to_binary32(Fraction(accs[g])) * sv[g]))
            assert Fraction(float(y8[m, n])) == X.round_to_binary32(t * sxv), (m, n)


ALL_RNG = (check_bf16_rounding, check_quantizer_exact, check_no_min_code, check_negation,
           check_matches_dequantize_then_matmul, check_q8_matches_dequantize_then_matmul,
           check_grouped_w4a8_exact, check_w4a16_exact, check_batch_invariant_rows,
           check_dynamic_w4a8, check_zero_points_reduce_to_symmetric, check_zero_points_exact,
           check_w8_float_exact, check_abs_terms_exact)
ALL_PLAIN = (check_hand_example_w4a32, check_q8_hand_example, check_hand_example_w4a8,
             check_hand_example_w4a16, check_every_nibble_code, check_f16_scales_decode_exactly,
             check_bf16_decode, check_pack_roundtrip, check_odd_k_pad, check_quantizer_ties,
             check_all_extreme, check_index_probe, check_shape_errors, check_error_measures,
             check_zero_points_closed_forms, check_q8_hand_example_float_activations,
             check_quantize_matrix, check_abs_terms_closed_form)


def run_all(seed=1234):
    """Run every pin; returns the list of names that failed."""
    failed = []
    for fn in ALL_PLAIN:
        try:
            fn()
        except Exception as e:  # noqa: BLE001 - any failure counts
            failed.append((fn.__name__, repr(e)[:200]))
    for fn in ALL_RNG:
        try:
            fn(np.random.default_rng(seed))
        except Exception as e:  # noqa: BLE001
            failed.append((fn.__name__, repr(e)[:200]))
    return failed
