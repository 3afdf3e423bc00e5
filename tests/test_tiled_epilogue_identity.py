"""Host check of the identity the tiled grouped W4A8 kernel's epilogue uses
(CPU only).

Each group's int8 MFMA sum starts from the bits of c = 1.5 * 2^19
(0x49400000) instead of 0 when it counts 16*acc, and from the bits of
c = 1.5 * 2^23 (0x4B400000) when it counts acc (zero points).  The i32 sum's
bits are then those of the binary32 F = c + acc, and the kernel forms
(F - c) * s in binary32, relying on F - c being f32(acc) exactly, so that
the product is the once-rounded f32(acc) * s of the grouped epilogue, bit
for bit, for every scale.  This test replays both sides in numpy binary32
over every accumulator the kernel can produce and a spread of scales:
bf16-valued, arbitrary f32, negative, subnormal, tiny, huge, infinite, NaN
and zero.
"""
import numpy as np

C16_BITS = 0x49400000   # 1.5 * 2^19: the sum counts 16 acc in units of 2^-4
C1_BITS = 0x4B400000    # 1.5 * 2^23: the sum counts acc in units of 1


def _both(c_bits, acc_sum, acc_true, s):
    F = (np.int64(c_bits) + acc_sum.astype(np.int64)).astype(np.int32).view(np.float32)
    c = np.array([c_bits], np.uint32).view(np.float32)[0]
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        fast = ((F - c).astype(np.float32)[:, None] * s[None, :]).astype(np.float32)
        want = (acc_true.astype(np.float32)[:, None] * s[None, :]).astype(np.float32)
    return fast, want


def _scales(rng):
    bf = (rng.uniform(0.002, 0.03, 200).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    anyf = rng.uniform(-1, 1, 200).astype(np.float32) * np.exp2(rng.integers(-126, 127, 200)).astype(np.float32)
    sub = np.array([1e-45, 3e-42, -7e-40, 1.17e-38, -1.0e-38, 2.0 ** -149, 2.0 ** -130], np.float32)
    big = np.array([2.0 ** 105, -(2.0 ** 105) * 1.75, 3.4e38, -3.4e38, 2.0 ** 127, 1.0, -1.0, 0.0, -0.0,
                    np.inf, -np.inf, np.nan], np.float32)
    return np.concatenate([bf, anyf, sub, big]).astype(np.float32)


def _same(a, b):
    """Bitwise equal, NaN payloads aside (both NaN counts as equal)."""
    return np.array_equal(a.view(np.uint32), b.view(np.uint32)) or (
        np.array_equal(np.isnan(a), np.isnan(b)) and
        np.array_equal(a[~np.isnan(a)].view(np.uint32), b[~np.isnan(b)].view(np.uint32)))


def test_identity_every_accumulator_sixteen_q():
    rng = np.random.default_rng(5)
    s = _scales(rng)
    lim = 128 * 127 * 128 // 16            # |acc_g| <= 130048 for codes -8..7, |x| <= 127 (16 q: -128..112)
    for lo in range(-lim, lim + 1, 8192):
        acc = np.arange(lo, min(lo + 8192, lim + 1), dtype=np.int64)
        fast, want = _both(C16_BITS, 16 * acc, acc, s)
        assert _same(fast, want), lo


def test_identity_every_accumulator_zero_points():
    rng = np.random.default_rng(6)
    s = _scales(rng)
    lim = 128 * 127 * 15                    # |acc_g| for u - z in -15..15
    for lo in range(-lim, lim + 1, 16384):
        acc = np.arange(lo, min(lo + 16384, lim + 1), dtype=np.int64)
        fast, want = _both(C1_BITS, acc, acc, s)
        assert _same(fast, want), lo


def test_start_value_keeps_every_sum_in_one_binade():
    """The sums stay inside c's binade, where F - c is exact."""
    for c_bits, unit, extreme, lo, hi in ((C16_BITS, 16, 128 * 127 * 128 // 16, 2.0 ** 19, 2.0 ** 20),
                                          (C1_BITS, 1, 128 * 127 * 15, 2.0 ** 23, 2.0 ** 24)):
        c = np.array([c_bits], np.uint32).view(np.float32)[0]
        for v in (-extreme, extreme):
            F = np.array([c_bits + unit * v], np.int32).view(np.float32)[0]
            assert lo <= F < hi
            assert float(F) - float(c) == v
