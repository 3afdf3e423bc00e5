"""The C ABI on the CPU: exports, host quantizers, and argument checking.

No GPU is needed: the host calls are plain C++, and every rejected device
call returns before its first HIP call.  Output canaries show that a
rejected call writes nothing ("Fused int4 and int8 dequantize-matmul in C",
tests table: shape_and_argument_errors leaves y untouched).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import int4_dequantize_matmul_amd as q4
import oracle.formats as F
import oracle.quantize as Q
from int4_dequantize_matmul_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "q4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q[48]_\w+)\s*\(", src)))


def test_library_exports_every_header_symbol():
    names = header_functions()
    assert "q4_linear_w4a8" in names and len(names) >= 14
    lib = q4.raw()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(q4.EXPORTS)


def test_probe_library_exports_and_checks():
    """libq4_probe (the benchmark's ceilings): every include/q4_probe.h call is
    exported and bound, and bad arguments return EINVAL before any launch."""
    from int4_dequantize_matmul_amd import probe
    src = open(os.path.join(ROOT, "include", "q4_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(q4_probe_\w+)\s*\(", src)))
    assert names and set(names) == set(probe.EXPORTS)
    lib = probe.raw()
    buf = (ctypes.c_uint8 * 64)()
    sink = (ctypes.c_uint32 * 4)()
    p, ps = ctypes.addressof(buf), ctypes.addressof(sink)
    p16 = (p + 15) & ~15
    assert lib.q4_probe_read(None, 16, ps, 1, 64, None) == q4.EINVAL
    assert lib.q4_probe_read(p16, 0, ps, 1, 64, None) == q4.EINVAL
    assert lib.q4_probe_read(p16 + 1, 16, ps, 1, 64, None) == q4.EINVAL
    assert lib.q4_probe_read(p16, 24, ps, 1, 64, None) == q4.EINVAL
    assert lib.q4_probe_read(p16, 16, ps, 0, 64, None) == q4.EINVAL
    assert lib.q4_probe_read(p16, 16, ps, 1, 96, None) == q4.EINVAL
    assert lib.q4_probe_read(p16, 32, p16 + 16, 1, 64, None) == q4.EINVAL   # sink inside buf
    assert lib.q4_probe_mfma_i8(None, 1, 1, None) == q4.EINVAL
    assert lib.q4_probe_mfma_i8(ps, 0, 1, None) == q4.EINVAL
    assert lib.q4_probe_mfma_i8(ps, 1, 0, None) == q4.EINVAL


def test_status_strings():
    for st in (0, 1, 2, 3, 4):
        assert q4.q4_status_string(st)
    assert q4.q4_status_string(99) == "unknown status"


def test_host_quantizer_matches_oracle_worked_cases():
    w = np.array([7, .5, 1.5, 2.5, -.5, -1.5, -2.5], np.float32)
    packed, s = q4.q4_quantize_row(w)
    assert s == 1.0 and packed.tolist() == [0x8F, 0xAA, 0x68, 0x86]
    q, s8 = q4.q8_quantize_row(np.array([889, 45.5, -45.5, 0.5], np.float32))
    assert s8 == 7.0 and q.tolist() == [127, 6, -6, 0]
    p0, s0 = q4.q4_quantize_row(np.zeros(3, np.float32))
    assert s0 == 0 and p0.tolist() == [0x88, 0x88]


def test_host_quantizer_bytes_equal_oracle_on_channel_workload():
    d = WL.w4a8_channel()
    W = d["W"]                             # all 3072 rows of K = 1023
    p_lib, s_lib = q4.q4_quantize_matrix(W)
    p_ref, s_ref = Q.quantize_q4_matrix(W)
    assert np.array_equal(p_lib, p_ref)
    assert np.array_equal(s_lib.view(np.uint32), s_ref.view(np.uint32))
    for m in range(d["M"]):
        ql, sl = q4.q8_quantize_row(d["x"][m])
        qr, sr = Q.quantize_q8_row(d["x"][m])
        assert np.array_equal(ql, qr) and sl.view(np.uint32) == sr.view(np.uint32)


def test_host_quantizer_bytes_equal_oracle_on_microdecoder_stack():
    """Every weight matrix of the microdecoder stack (35 linears, 257M
    weights), byte for byte and scale bit for scale bit."""
    for i in range(len(WL.microdecoder_linears())):
        W = WL.microdecoder_linear(i)["W"]
        p_lib, s_lib = q4.q4_quantize_matrix(W)
        p_ref, s_ref = Q.quantize_q4_matrix(W)
        assert np.array_equal(p_lib, p_ref), i
        assert np.array_equal(s_lib.view(np.uint32), s_ref.view(np.uint32)), i


def test_host_quantizer_random_rows_and_ties():
    rng = np.random.default_rng(5)
    for K in (1, 2, 7, 64, 1023, 4097, 9000):
        w = (rng.standard_normal(K) * np.exp2(rng.integers(-10, 10))).astype(np.float32)
        w[rng.integers(0, K)] = np.float32(3.5) * (np.abs(w).max() / np.float32(7))
        p_lib, s_lib = q4.q4_quantize_row(w)
        p_ref, s_ref = Q.quantize_q4_row(w)
        assert np.array_equal(p_lib, p_ref) and s_lib == s_ref, K
        q_lib, t_lib = q4.q8_quantize_row(w)
        q_ref, t_ref = Q.quantize_q8_row(w)
        assert np.array_equal(q_lib, q_ref) and t_lib == t_ref, K


def test_host_quantizer_rejects_non_finite():
    lib = q4.raw()
    w = np.array([1.0, np.nan], np.float32)
    out = np.full(1, 0xAB, np.uint8)
    s = np.full(1, 7.0, np.float32)
    assert lib.q4_quantize_row(w.ctypes.data, 2, out.ctypes.data, s.ctypes.data) == q4.EINVAL
    assert out[0] == 0xAB and s[0] == 7.0
    assert lib.q4_quantize_row(None, 2, out.ctypes.data, s.ctypes.data) == q4.EINVAL
    assert lib.q4_quantize_row(w.ctypes.data, -1, out.ctypes.data, s.ctypes.data) == q4.EINVAL


def test_pack_matches_oracle_both_encodings():
    rng = np.random.default_rng(9)
    for K in (1, 2, 3, 64, 65):
        codes = rng.integers(-8, 8, (7, K))
        for enc in F.ENCODINGS:
            assert np.array_equal(q4.q4_pack(codes, enc), F.pack_codes(codes, enc)), (K, enc)
    with pytest.raises(q4.Q4Error):
        q4.q4_pack(np.array([[8]]), "excess8")


# --------------------------------------------------------------------------
# device entry points: rejected before any HIP call
# --------------------------------------------------------------------------

class Canary:
    """Host buffers standing in for device buffers; rejected calls never
    dereference them, so their bytes must come back unchanged."""

    def __init__(self, nbytes=4096):
        self.a = np.full(nbytes, 0x5A, np.uint8)

    @property
    def p(self):
        return ctypes.c_void_p(self.a.ctypes.data)

    def untouched(self):
        return bool(np.all(self.a == 0x5A))


def _bufs(n=6):
    return [Canary() for _ in range(n)]


def test_w4a32_argument_errors():
    lib = q4.raw()
    x, w, s, y = _bufs(4)
    f = lib.q4_linear_w4a32
    ok = (x.p, w.p, s.p, y.p)
    assert f(None, w.p, s.p, y.p, 1, 2, 4, 2, 0, None) == q4.EINVAL
    assert f(x.p, None, s.p, y.p, 1, 2, 4, 2, 0, None) == q4.EINVAL      # NULL weights (mutant s11)
    assert f(*ok, -1, 2, 4, 2, 0, None) == q4.EINVAL
    assert f(*ok, 1, 2, 4, 2, 7, None) == q4.EINVAL                      # unknown encoding
    assert f(x.p, w.p, s.p, None, 0, 0, 0, 2, 0, None) == q4.EINVAL      # NULL even with empty dims
    for K, G in ((3, 1), (4, 3), (4, 0), (4, -2), (8, 6), (6, 4)):       # mutant s10: G must divide K
        assert f(*ok, 1, 2, K, G, 0, None) == q4.ESHAPE, (K, G)
    assert f(*ok, 0, 2, 4, 2, 0, None) == q4.OK                          # empty: no-op
    assert f(*ok, 1, 0, 4, 2, 0, None) == q4.OK
    assert f(x.p, w.p, s.p, x.p, 1, 2, 4, 2, 0, None) == q4.EINVAL       # y overlaps x
    assert all(b.untouched() for b in (x, w, s, y))


def test_w4a16_argument_errors():
    lib = q4.raw()
    x, w, s, yb, yf = _bufs(5)
    f = lib.q4_linear_w4a16
    assert f(x.p, w.p, s.p, None, yf.p, 1, 2, 4, 2, 1, None) == q4.EINVAL   # y_bf16 required
    assert f(x.p, w.p, s.p, yb.p, yb.p, 1, 2, 4, 2, 1, None) == q4.EINVAL   # outputs overlap
    assert f(x.p, w.p, s.p, yb.p, None, 1, 2, 5, 5, 1, None) == q4.ESHAPE
    assert f(x.p, w.p, s.p, yb.p, None, 0, 2, 4, 2, 1, None) == q4.OK
    assert all(b.untouched() for b in (x, w, s, yb, yf))


def test_w4a8_argument_errors():
    lib = q4.raw()
    xq, sx, w, sw, y = _bufs(5)
    f = lib.q4_linear_w4a8
    args = (xq.p, sx.p, w.p, sw.p, y.p)
    assert f(xq.p, None, w.p, sw.p, y.p, 1, 2, 4, 0, 1, None) == q4.EINVAL
    assert f(*args, 1, 2, 4, -2, 1, None) == q4.EINVAL                   # negative G
    assert f(*args, 1, 2, 6, 4, 1, None) == q4.ESHAPE                    # G does not divide K
    assert f(*args, 1, 2, 5, 2, 1, None) == q4.ESHAPE                    # grouped needs even K
    assert f(*args, 1, 2, q4.W4A8_MAX_K + 2, 0, 1, None) == q4.ESHAPE   # i32 overflow bound
    assert f(*args, 0, 2, 1023, 0, 1, None) == q4.OK                     # odd K fine per channel
    assert f(xq.p, sx.p, w.p, sw.p, sw.p, 1, 2, 4, 0, 1, None) == q4.EINVAL  # y overlaps sw
    assert all(b.untouched() for b in (xq, sx, w, sw, y))


def test_zero_point_argument_errors():
    """The zero-point entry points: zeros is a required input checked for
    overlap like the others; per-channel zero points do not exist (ESHAPE)."""
    lib = q4.raw()
    x, w, s, z, yb, yf = _bufs(6)
    f = lib.q4_linear_w4a16_zp
    assert f(x.p, w.p, s.p, None, yb.p, None, 1, 2, 4, 2, None) == q4.EINVAL      # zeros required
    assert f(x.p, w.p, s.p, z.p, None, yf.p, 1, 2, 4, 2, None) == q4.EINVAL      # y_bf16 required
    assert f(x.p, w.p, s.p, z.p, z.p, None, 1, 2, 4, 2, None) == q4.EINVAL       # y overlaps zeros
    assert f(x.p, w.p, s.p, z.p, yb.p, None, 1, 2, 5, 5, None) == q4.ESHAPE
    assert f(x.p, w.p, s.p, z.p, yb.p, None, 0, 2, 4, 2, None) == q4.OK
    xq, sx, sw, y = _bufs(4)
    g = lib.q4_linear_w4a8_zp
    assert g(xq.p, sx.p, w.p, sw.p, None, y.p, 1, 2, 4, 2, None) == q4.EINVAL     # zeros required
    assert g(xq.p, sx.p, w.p, sw.p, z.p, z.p, 1, 2, 4, 2, None) == q4.EINVAL      # y overlaps zeros
    assert g(xq.p, sx.p, w.p, sw.p, z.p, y.p, 1, 2, 4, 0, None) == q4.ESHAPE      # per channel: no groups
    assert g(xq.p, sx.p, w.p, sw.p, z.p, y.p, 1, 2, 6, 4, None) == q4.ESHAPE      # G does not divide K
    assert g(xq.p, sx.p, w.p, sw.p, z.p, y.p, 1, 2, 4, -2, None) == q4.EINVAL     # negative G
    assert g(xq.p, sx.p, w.p, sw.p, z.p, y.p, 0, 2, 4, 2, None) == q4.OK
    assert all(b.untouched() for b in (x, w, s, z, yb, yf, xq, sx, sw, y))


def test_w8_float_argument_errors():
    lib = q4.raw()
    x, w, s, y, yb = _bufs(5)
    assert lib.q8_linear_w8a32(None, w.p, s.p, y.p, 1, 2, 4, None) == q4.EINVAL
    assert lib.q8_linear_w8a32(x.p, w.p, s.p, x.p, 1, 2, 4, None) == q4.EINVAL      # y overlaps x
    assert lib.q8_linear_w8a32(x.p, w.p, s.p, y.p, -1, 2, 4, None) == q4.EINVAL
    assert lib.q8_linear_w8a32(x.p, w.p, s.p, y.p, 0, 2, 4, None) == q4.OK
    assert lib.q8_linear_w8a16(x.p, w.p, s.p, None, y.p, 1, 2, 4, None) == q4.EINVAL  # y_bf16 required
    assert lib.q8_linear_w8a16(x.p, w.p, s.p, yb.p, yb.p, 1, 2, 4, None) == q4.EINVAL  # outputs overlap
    assert lib.q8_linear_w8a16(x.p, w.p, s.p, yb.p, None, 1, 0, 4, None) == q4.OK
    assert all(b.untouched() for b in (x, w, s, y, yb))


def test_w8a8_and_quantize_rows_argument_errors():
    lib = q4.raw()
    xq, sx, w, sw, y, x = _bufs(6)
    assert lib.q8_linear_w8a8(xq.p, sx.p, w.p, sw.p, y.p, 1, 2, q4.W8A8_MAX_K + 1, None) == q4.ESHAPE
    assert lib.q8_linear_w8a8(xq.p, sx.p, None, sw.p, y.p, 1, 2, 4, None) == q4.EINVAL
    assert lib.q8_quantize_rows(x.p, 5, 1, 4, xq.p, sx.p, None) == q4.EINVAL   # unknown dtype
    assert lib.q8_quantize_rows(x.p, 0, 1, 4, x.p, sx.p, None) == q4.EINVAL    # xq overlaps x
    assert lib.q8_quantize_rows(x.p, 0, 0, 4, xq.p, sx.p, None) == q4.OK
    assert all(b.untouched() for b in (xq, sx, w, sw, y, x))


def test_dynamic_workspace_rules():
    lib = q4.raw()
    assert q4.q4_w4a8_dynamic_workspace(4, 1023) == 4096 + 256
    assert q4.q4_w4a8_dynamic_workspace(0, 0) == 0
    x, w, sw, y = _bufs(4)
    ws = np.zeros(8192 + 512, np.uint8)
    base = (ws.ctypes.data + 255) & ~255
    f = lib.q4_linear_w4a8_dynamic
    need = q4.q4_w4a8_dynamic_workspace(4, 16)
    assert f(x.p, 0, w.p, sw.p, y.p, 4, 2, 16, 0, 1, ctypes.c_void_p(base), need - 1, None) == q4.EINVAL
    assert f(x.p, 0, w.p, sw.p, y.p, 4, 2, 16, 0, 1, ctypes.c_void_p(base + 4), need, None) == q4.EINVAL
    assert f(x.p, 0, w.p, sw.p, y.p, 0, 2, 16, 0, 1, ctypes.c_void_p(base), need, None) == q4.OK
    assert all(b.untouched() for b in (x, w, sw, y))


def test_noalloc_argument_rules():
    """The no-allocation dynamic call: the workspace checks are gone, the
    others are those of the workspace call, and a size whose workspace would
    exceed the library's scratch array is ESHAPE; all before any HIP call."""
    lib = q4.raw()
    x, w, sw, y = _bufs(4)
    f = lib.q4_linear_w4a8_dynamic_noalloc
    assert f(None, 0, w.p, sw.p, y.p, 4, 2, 16, 0, 1, None) == q4.EINVAL
    assert f(x.p, 7, w.p, sw.p, y.p, 4, 2, 16, 0, 1, None) == q4.EINVAL          # unknown dtype
    assert f(x.p, 0, w.p, sw.p, x.p, 4, 2, 16, 0, 1, None) == q4.EINVAL          # y overlaps x
    assert f(x.p, 0, w.p, sw.p, y.p, -1, 2, 16, 0, 1, None) == q4.EINVAL
    assert f(x.p, 0, w.p, sw.p, y.p, 4, 2, 15, 128, 1, None) == q4.ESHAPE        # grouped shape rule
    big_m = q4.NOALLOC_SCRATCH_BYTES // 1024 + 1
    assert q4.q4_w4a8_dynamic_workspace(big_m, 1024) > q4.NOALLOC_SCRATCH_BYTES
    # buffers of the sizes the call declares, so that no range overlaps another
    xb = np.zeros(big_m * 1024 * 4, np.uint8)
    yb = np.zeros(big_m * 2 * 4, np.uint8)
    assert f(ctypes.c_void_p(xb.ctypes.data), 0, w.p, sw.p, ctypes.c_void_p(yb.ctypes.data),
             big_m, 2, 1024, 0, 1, None) == q4.ESHAPE
    assert not xb.any() and not yb.any()
    assert f(x.p, 0, w.p, sw.p, y.p, 0, 2, 16, 0, 1, None) == q4.OK
    assert all(b.untouched() for b in (x, w, sw, y))


def test_path_override():
    assert q4.q4_get_path() == "auto"
    for p in ("generic", "gemv", "tiled", "gemv_mc", "auto"):
        q4.q4_set_path(p)
        assert q4.q4_get_path() == p
    assert q4.raw().q4_set_path(9) == q4.EINVAL


def test_multi_argument_errors():
    lib = q4.raw()
    x, w, s, y, y2 = (Canary(1 << 18) for _ in range(5))
    f = lib.q4_linear_w4a8_dynamic_multi

    def probs(*rows):
        arr = (q4.W4A8Problem * max(len(rows), 1))()
        for i, (xp, wp, sp, yp, N, K) in enumerate(rows):
            arr[i] = q4.W4A8Problem(xp.value if xp else None, wp.value if wp else None,
                                    sp.value if sp else None, yp.value if yp else None, N, K)
        return arr

    good = (x.p, w.p, s.p, y.p, 16, 64)
    one = probs(good)
    bf16 = q4.DT["bf16"]
    assert f(one, -1, bf16, 1, None) == q4.EINVAL
    assert f(probs(*[good] * 65), 65, bf16, 1, None) == q4.EINVAL          # more than Q4_MULTI_MAX
    assert f(None, 1, bf16, 1, None) == q4.EINVAL
    assert f(None, 0, bf16, 1, None) == q4.OK                              # nothing to do
    assert f(one, 1, 7, 1, None) == q4.EINVAL                              # unknown dtype
    assert f(one, 1, bf16, -1, None) == q4.EINVAL
    assert f(probs((None, w.p, s.p, y.p, 16, 64)), 1, bf16, 1, None) == q4.EINVAL
    assert f(probs((x.p, w.p, s.p, y.p, -1, 64)), 1, bf16, 1, None) == q4.EINVAL
    w4 = ctypes.c_void_p(w.p.value + 4)
    assert f(probs((x.p, w4, s.p, y.p, 16, 64)), 1, bf16, 1, None) == q4.EINVAL     # wq not 16-byte aligned
    assert f(probs((x.p, w.p, s.p, x.p, 16, 64)), 1, bf16, 1, None) == q4.EINVAL    # y over its own x
    assert f(probs(good, (y.p, w.p, s.p, y2.p, 16, 64)), 2, bf16, 1, None) == q4.EINVAL  # y over another x
    assert f(probs(good, (x.p, w.p, s.p, y.p, 16, 64)), 2, bf16, 1, None) == q4.EINVAL  # two outputs share y
    assert f(one, 1, bf16, 17, None) == q4.ESHAPE                          # M > 16
    assert f(probs((x.p, w.p, s.p, y.p, 16, 30)), 1, bf16, 1, None) == q4.ESHAPE   # ceil(K/2) % 16 != 0
    assert f(probs((x.p, w.p, s.p, y.p, 1, 63488 + 2048)), 1, bf16, 1, None) == q4.ESHAPE  # LDS at M = 1
    assert f(probs((x.p, w.p, s.p, y.p, 1, 4096)), 1, bf16, 16, None) == q4.ESHAPE        # LDS at M = 16
    assert f(one, 1, bf16, 0, None) == q4.OK                               # M == 0: no-op
    assert all(b.untouched() for b in (x, w, s, y, y2))


def test_selftest_argument_errors():
    """The selftest needs a caller workspace of the stated size, 256-byte
    aligned; anything else is EINVAL before any HIP call."""
    lib = q4.raw()
    need = lib.q4_selftest_workspace()
    assert 12 << 20 <= need <= 13 << 20
    buf = np.zeros(need + 512, np.uint8)
    base = (buf.ctypes.data + 255) & ~255
    assert lib.q4_selftest(None, need, None) == q4.EINVAL
    assert lib.q4_selftest(ctypes.c_void_p(base + 16), need, None) == q4.EINVAL
    assert lib.q4_selftest(ctypes.c_void_p(base), need - 1, None) == q4.EINVAL
    assert lib.q4_selftest_report()


def test_header_is_plain_c():
    """include/q4.h is a C header: it compiles as C99 with every warning on."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c",
                        os.path.join(ROOT, "include", "q4.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
