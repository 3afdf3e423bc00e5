"""Host check of the identity the tiled grouped W4A8 kernel's epilogue uses
(CPU only).

Each group's int8 MFMA sum starts from the bits of c = 1/(2 pi) (0x3E22F983)
instead of 0, so the i32 sum of 16*acc (or acc with zero points) has the
bits of the binary32 F = c + 16*acc*2^-26.  The kernel then forms
(F - c) * (s * 2^22) (or * 2^26) in binary32 and relies on that being the
once-rounded product f32(acc) * s of the grouped epilogue, bit for bit.
This test replays both sides in numpy binary32 over every accumulator the
kernel can produce and a spread of scales: bf16-valued, arbitrary f32,
negative, subnormal, tiny, huge (up to the 2^106 limit the kernel flags),
and zero.
"""
import numpy as np

C_BITS = 0x3E22F983


def _both(acc_sum, acc_true, s, factor):
    F = (np.int64(C_BITS) + acc_sum.astype(np.int64)).astype(np.int32).view(np.float32)
    c = np.array([C_BITS], np.uint32).view(np.float32)[0]
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        sa = (s * np.float32(factor)).astype(np.float32)
        fast = ((F - c).astype(np.float32)[:, None] * sa[None, :]).astype(np.float32)
        want = (acc_true.astype(np.float32)[:, None] * s[None, :]).astype(np.float32)
    return fast, want, sa


def _scales(rng):
    bf = (rng.uniform(0.002, 0.03, 200).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    anyf = rng.uniform(-1, 1, 200).astype(np.float32) * np.exp2(rng.integers(-126, 100, 200)).astype(np.float32)
    sub = np.array([1e-45, 3e-42, -7e-40, 1.17e-38, -1.0e-38, 2.0 ** -149, 2.0 ** -130], np.float32)
    big = np.array([2.0 ** 105, -(2.0 ** 105) * 1.75, 3.4e31, 1.0, -1.0, 0.0, -0.0], np.float32)
    return np.concatenate([bf, anyf, sub, big]).astype(np.float32)


def test_identity_every_accumulator_sixteen_q():
    rng = np.random.default_rng(5)
    s = _scales(rng)
    lim = 128 * 127 * 128 // 16            # |acc_g| <= 130048 for codes -8..7, |x| <= 127 (16 q: -128..112)
    for lo in range(-lim, lim + 1, 8192):
        acc = np.arange(lo, min(lo + 8192, lim + 1), dtype=np.int64)
        fast, want, sa = _both(16 * acc, acc, s, 2.0 ** 22)
        ok = np.isfinite(sa) | ~np.isfinite(s)            # the kernel flags steps with sa overflowing
        assert np.array_equal(fast[:, ok].view(np.uint32), want[:, ok].view(np.uint32)), lo


def test_identity_every_accumulator_zero_points():
    rng = np.random.default_rng(6)
    s = _scales(rng)
    lim = 128 * 127 * 15                    # |acc_g| for u - z in -15..15
    for lo in range(-lim, lim + 1, 16384):
        acc = np.arange(lo, min(lo + 16384, lim + 1), dtype=np.int64)
        fast, want, sa = _both(acc, acc, s, 2.0 ** 26)
        ok = np.isfinite(sa) | ~np.isfinite(s)
        assert np.array_equal(fast[:, ok].view(np.uint32), want[:, ok].view(np.uint32)), lo


def test_start_value_keeps_every_sum_in_one_binade():
    """The sums stay inside c's binade, where F - c is exact."""
    c = np.array([C_BITS], np.uint32).view(np.float32)[0]
    for extreme in (128 * 127 * 128, 128 * 127 * 15):
        for v in (-extreme, extreme):
            F = np.array([C_BITS + v], np.int32).view(np.float32)[0]
            assert 0.125 <= F < 0.25
            assert float(F) - float(c) == v * 2.0 ** -26
