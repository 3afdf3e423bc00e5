"""GPU parity: the HIP path against the oracle on the same seeded inputs.

Integer-activation paths (W4A8, W8A8, the activation quantizer) must match
bit for bit.  Float-activation paths are judged against the float64 oracle:
normwise and conditioned relative error <= 1e-5 for f32 output and <= 2e-2
for bf16 output; the bf16 output must also equal the round-to-nearest-even
of the f32 output bit for bit.

Every route is exercised (generic, decode GEMV, and the tiled kernels where
a shape allows them) at sizes that span several tiles with ragged tails, and
at the workloads' full sizes in the launch configuration the bench times.
"""
import functools

import numpy as np
import pytest
import torch

import int4_dequantize_matmul_amd as q4
import oracle.formats as F
import oracle.linear as L
import oracle.quantize as Q
from int4_dequantize_matmul_amd import workloads as WL
from tests.gpu_util import assert_bitwise, assert_close, dev, host

pytestmark = pytest.mark.gpu
F32_TOL, BF16_TOL = 1e-5, 2e-2


@pytest.fixture(autouse=True)
def _auto_path():
    q4.q4_set_path("auto")
    yield
    q4.q4_set_path("auto")


def _paths(*names):
    return pytest.mark.parametrize("path", names)


# --------------------------------------------------------------------------
# worked example ("Fused int4 and int8 dequantize-matmul in C", section 3)
# --------------------------------------------------------------------------

@_paths("generic", "gemv", "auto")
def test_worked_example_every_linear(path):
    q4.q4_set_path(path)
    codes = np.array([[1, -2, 3, -8], [7, 0, -1, 4]])
    x = np.array([[1, 2, 3, 4]], np.float32)
    # W4A32, two's complement, f16 scales 0.5 2 / 1 0.25
    y = q4.q4_linear_w4a32(dev(x), dev(F.pack_codes(codes, F.TWOS)),
                           dev(np.array([[0x3800, 0x4000], [0x3C00, 0x3400]], np.uint16), torch.float16), 2)
    assert host(y).tolist() == [[-47.5, 10.25]]
    # W4A16 with bf16 x and scales, both encodings
    for enc in F.ENCODINGS:
        yb, yf = q4.q4_linear_w4a16(dev(np.array([[0x3F80, 0x4000, 0x4040, 0x4080]], np.uint16)),
                                    dev(F.pack_codes(codes, enc)),
                                    dev(np.array([[0x3F00, 0x4000], [0x3F80, 0x3E80]], np.uint16)), 2, enc,
                                    want_f32=True)
        assert host(yf).tolist() == [[-47.5, 10.25]]
        assert host(yb).tolist() == [[0xC23E, 0x4124]]   # bf16 of -47.5 and 10.25
    xq = dev(np.array([[1, 2, 3, 4]], np.int8))
    one = dev(np.array([1.0], np.float32))
    # W4A8 per channel, scales 0.5 / 0.25 -> [-13, 5]; grouped -> [-47.5, 10.25]
    for enc in F.ENCODINGS:
        p = dev(F.pack_codes(codes, enc))
        y = q4.q4_linear_w4a8(xq, one, p, dev(np.array([0.5, 0.25], np.float32)), 0, enc)
        assert host(y).tolist() == [[-13.0, 5.0]]
        y = q4.q4_linear_w4a8(xq, one, p, dev(np.array([[0.5, 2.0], [1.0, 0.25]], np.float32)), 2, enc)
        assert host(y).tolist() == [[-47.5, 10.25]]
    y = q4.q8_linear_w8a8(xq, one, dev(codes.astype(np.int8)), dev(np.array([0.5, 0.25], np.float32)))
    assert host(y).tolist() == [[-13.0, 5.0]]


# --------------------------------------------------------------------------
# activation quantizer
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,bf16", [(4, 1023, False), (3, 2048, True), (5, 8, False), (2, 5632, True),
                                      (1, 1, False), (7, 9000, False)])
def test_quantize_rows_bitwise(M, K, bf16):
    rng = np.random.default_rng(M * 1000 + K)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[0, : min(K, 3)] = 0.0
    if M > 2:
        x[2] = 0.0                                        # an all-zero row
    if K >= 8:   # plant exact ties: |x|max/127 = 7 exactly, 45.5 / 7 = 6.5
        x[-1, 0], x[-1, 1] = np.float32(889.0), np.float32(45.5)
    xin = WL.bf16_bits(x) if bf16 else x
    xq, sx = q4.q8_quantize_rows(dev(xin))
    xq_ref, sx_ref = Q.quantize_q8_rows(xin, "bf16" if bf16 else "f32")
    assert_bitwise(host(xq), xq_ref, "xq")
    assert_bitwise(host(sx), sx_ref, "sx")


def test_quantize_rows_prefill_activations_bitwise():
    d = WL.w4a8_prefill()
    xq, sx = q4.q8_quantize_rows(dev(d["x"]))
    xq_ref, sx_ref = Q.quantize_q8_rows(d["x"], "bf16")
    assert_bitwise(host(xq), xq_ref, "xq")
    assert_bitwise(host(sx), sx_ref, "sx")


# --------------------------------------------------------------------------
# W4A8 and W8A8 (bit-exact)
# --------------------------------------------------------------------------

@_paths("generic", "gemv", "auto")
def test_w4a8_channel_workload_bitwise(path):
    """M=4, N=3072, K=1023 (odd K, pad nibble) end to end: host quantizer,
    device activation quantizer, W4A8 linear."""
    q4.q4_set_path(path)
    d = WL.w4a8_channel()
    packed, sw = q4.q4_quantize_matrix(d["W"])
    p_ref, sw_ref = Q.quantize_q4_matrix(d["W"])
    assert_bitwise(packed, p_ref, "packed")
    assert_bitwise(sw, sw_ref, "scales")
    y = q4.q4_linear_w4a8_dynamic(dev(d["x"]), dev(packed), dev(sw), 0, "excess8")
    y_ref, xq_ref, sx_ref = L.linear_w4a8_dynamic(d["x"], p_ref, sw_ref, 0, F.EXCESS8, "f32")
    assert_bitwise(host(y), y_ref, f"y via {q4.q4_last_path()}")


W4A8_CASES = [  # M, N, K, G
    (1, 37, 256, 128), (4, 80, 384, 128), (16, 128, 1024, 256), (17, 45, 512, 128),
    (40, 96, 256, 0), (3, 33, 1023, 0), (2, 64, 130, 0), (5, 19, 2048, 0), (64, 130, 1024, 128),
    (1, 16, 128, 128), (9, 200, 768, 384),
    (16, 40, 4096, 0), (16, 40, 4096, 512), (12, 33, 8320, 0),   # several LDS slabs / generic
    (16, 40, 5632, 128), (7, 33, 8192, 128), (2, 24, 8192, 256),  # grouped GEMV past 64 KB of LDS
    (130, 200, 2048, 128), (129, 129, 128, 128), (256, 256, 384, 0),  # tiled: ragged tiles, one step
    (1, 70, 5632, 0), (4, 33, 4095, 0), (2, 20, 10240, 0), (8, 40, 2048, 0),  # streaming per-channel decode
]


@pytest.mark.parametrize("M,N,K,G", W4A8_CASES)
@pytest.mark.parametrize("enc", F.ENCODINGS)
@_paths("generic", "gemv", "tiled", "auto")
def test_w4a8_bitwise(M, N, K, G, enc, path):
    q4.q4_set_path(path)
    c = WL.small_int_case(M * 7 + N + K + G, M, N, K, G)
    y = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), G, enc)
    y_ref = L.linear_w4a8(c["xq"], c["sx"], c["w"], c["sw"], G, enc)
    assert_bitwise(host(y), y_ref, f"W4A8 M{M} N{N} K{K} G{G} {enc} via {q4.q4_last_path()}")


# shapes of the measured route plan: the microdecoder's q/k/v/o, gate/up and
# down linears and the prefill's gate_up linear
ROUTE_SHAPES = [(2048, 2048), (5632, 2048), (13312, 2048), (2048, 5632)]


def _route_ms(dmax):
    return sorted({1, 2, 16, 17, dmax, dmax + 1})


def _route_cols(N):
    return np.r_[0:192, N - 64:N]      # sampled output columns, both ends


@pytest.mark.parametrize("N,K", ROUTE_SHAPES)
@pytest.mark.parametrize("G", [0, 128])
def test_w4a8_route_by_batch(N, K, G):
    """The default route follows the measured plan: the decode kernels up to
    the shape's crossing, the tiled kernel from the next row; the call takes
    the route q4_route_plan names, and every route is bit-exact (sampled
    columns against the oracle)."""
    dmax = q4.q4_route_plan("w4a8", 1, N, K, G)["decode_max"]
    assert dmax >= 16
    cols = _route_cols(N)
    for M in _route_ms(dmax):
        want = "gemv" if M <= dmax else "tiled"
        assert q4.q4_route_plan("w4a8", M, N, K, G)["path"] == want, (M, N, K, G)
        c = WL.small_int_case(M * 7 + N + G, M, N, K, G)
        y = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), G, "excess8")
        assert q4.q4_last_path() == want, (M, N, K, G)
        y_ref = L.linear_w4a8(c["xq"], c["sx"], c["w"][cols], c["sw"][cols], G, F.EXCESS8)
        assert_bitwise(host(y)[:, cols], y_ref, f"M{M} N{N} K{K} G{G} via {want}")


@pytest.mark.parametrize("G", [2, 32, 64])
def test_w4a8_small_groups_bitwise(G):
    c = WL.small_int_case(G, 6, 37, 384, G)
    y = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), G, "twos")
    assert_bitwise(host(y), L.linear_w4a8(c["xq"], c["sx"], c["w"], c["sw"], G, F.TWOS), f"G{G}")


@pytest.mark.parametrize("M,N,K", [(1, 37, 200), (4, 64, 256), (16, 80, 1024), (23, 33, 64), (3, 17, 5632),
                                   (16, 33, 4096)])
@_paths("generic", "gemv", "auto")
def test_w8a8_bitwise(M, N, K, path):
    q4.q4_set_path(path)
    c = WL.small_int_case(M + N + K, M, N, K, 0, w_int8=True)
    y = q4.q8_linear_w8a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]))
    assert_bitwise(host(y), L.linear_w8a8(c["xq"], c["sx"], c["w"], c["sw"]), f"W8A8 via {q4.q4_last_path()}")


def test_w4a8_all_extreme_rows():
    """xq = +-127 against codes +-7 (per channel) and -8 (grouped): closed forms."""
    for K in (2048, 5632):
        xq = np.full((2, K), 127, np.int8)
        xq[1] = -127
        codes = np.full((16, K), 7)
        codes[1::2] = -7
        one = np.ones(2, np.float32)
        y = q4.q4_linear_w4a8(dev(xq), dev(one), dev(F.pack_codes(codes, F.EXCESS8)),
                              dev(np.ones(16, np.float32)), 0, "excess8")
        want = np.array([[889.0 * K, -889.0 * K] * 8, [-889.0 * K, 889.0 * K] * 8], np.float32)
        assert_bitwise(host(y), want, f"extreme K{K}")
        c8 = np.full((16, K), -8)
        y = q4.q4_linear_w4a8(dev(xq), dev(one), dev(F.pack_codes(c8, F.TWOS)),
                              dev(np.ones((16, K // 128), np.float32)), 128, "twos")
        assert_bitwise(host(y), np.array([[-1016.0 * K] * 16, [1016.0 * K] * 16], np.float32), "extreme g")


@_paths("generic", "gemv", "tiled")
def test_w4a8_grouped_tiny_scales_bitwise(path):
    """Group scales down to the f32 subnormals (and zero, and signs): the
    products and the running sum stay IEEE, with no flush to zero."""
    q4.q4_set_path(path)
    M, N, K, G = 40, 150, 512, 128
    c = WL.small_int_case(4242, M, N, K, G)
    sw = c["sw"].copy()
    tiny = np.array([0.0, 2.0 ** -125, -(2.0 ** -124) * 1.375, 1e-40, -3e-45, 2.0 ** -120,
                     1.1754942e-38, 7e-39], np.float32)
    sw[::3, 1] = tiny[np.arange(sw[::3].shape[0]) % tiny.size]
    sw[5, :] = 1e-41
    y = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(sw), G, "excess8")
    assert_bitwise(host(y), L.linear_w4a8(c["xq"], c["sx"], c["w"], sw, G, F.EXCESS8),
                   f"tiny scales via {q4.q4_last_path()}")


def _bf16_valued(a):
    """Round f32 values to the nearest bf16 value (ties to even), kept as f32."""
    return F.bf16_bits_to_f32(F.f32_to_bf16_bits(np.asarray(a, np.float32)))


@pytest.mark.parametrize("K", [384, 2176, 5120])
@pytest.mark.parametrize("zp", [False, True])
@pytest.mark.parametrize("misaligned", [False, True])
def test_w4a8_grouped_tiled_epilogue_forms(K, zp, misaligned):
    """The tiled kernel's two grouped epilogue forms in one launch, bit for
    bit against the oracle.  bf16-valued scales take the fast form (an fma
    with the exact c*s); one column in some waves has a scale that forces the
    plain form there: full f32 precision, zero, negative, or c*s overflowing.
    Subnormal and huge bf16 scales stay in the fast form.  K = 384 (3 groups),
    2176 (17) and 5120 (40) cover a wave's scale run below 1 KB, over several
    1 KB pieces and over two 4 KB rounds; misaligned scales take the plain
    form everywhere."""
    M, N, G = 200, 300, 128
    c = WL.small_int_case(9100 + K, M, N, K, G)
    sw = _bf16_valued(c["sw"])
    sw[7, 1] = np.nextafter(np.float32(0.0123), np.float32(1))   # 3 s not exact: plain form in that wave
    assert np.float64(np.float32(3.0) * sw[7, 1]) != 3.0 * np.float64(sw[7, 1])
    sw[200, 0] = 0.0                              # zero scale
    sw[290, -1] = -sw[290, -1]                    # negative scale
    sw[100, 2] = np.float32(3.0e38)               # c * s overflows
    sw[40, :] = _bf16_valued(np.float32(2.0 ** -130))   # subnormal, fast form
    sw[170, 1] = _bf16_valued(np.float32(2.0 ** 100))   # huge, fast form
    q4.q4_set_path("tiled")
    if misaligned:
        flat = dev(np.concatenate([np.zeros(1, np.float32), sw.reshape(-1)]))
        swd = flat[1:].view(N, K // G)
        assert swd.data_ptr() % 16 == 4
    else:
        swd = dev(sw)
    if zp:
        z = np.random.default_rng(9200 + K).integers(0, 16, (N, K // G), dtype=np.uint8)
        y = q4.q4_linear_w4a8_zp(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), swd, dev(z), G)
        ref = L.linear_w4a8_zp(c["xq"], c["sx"], c["w"], sw, z, G)
    else:
        y = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), swd, G, "excess8")
        ref = L.linear_w4a8(c["xq"], c["sx"], c["w"], sw, G, F.EXCESS8)
    assert q4.q4_last_path() == "tiled"
    assert_bitwise(host(y), ref, f"epilogue forms K={K} zp={zp} misaligned={misaligned}")


def test_w4a8_per_channel_largest_tiled_k():
    """K = 131072 with xq = +-127 against code -8: the tiled kernel's sums
    reach 16 * 127 * 8 * K = 2130706432 in magnitude, just inside i32."""
    M, N, K = 17, 16, 131072
    rng = np.random.default_rng(77)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int8)
    xq[0], xq[1] = 127, -127
    codes = rng.integers(-8, 8, (N, K))
    codes[0], codes[1] = -8, 7
    w = F.pack_codes(codes, F.EXCESS8)
    sx = rng.uniform(0.001, 0.02, M).astype(np.float32)
    sw = rng.uniform(0.001, 0.02, N).astype(np.float32)
    q4.q4_set_path("tiled")
    y = q4.q4_linear_w4a8(dev(xq), dev(sx), dev(w), dev(sw), 0, "excess8")
    assert q4.q4_last_path() == "tiled"
    assert_bitwise(host(y), L.linear_w4a8(xq, sx, w, sw, 0, F.EXCESS8), "K=131072")


@pytest.mark.parametrize("off", [1, 2, 3])
@pytest.mark.parametrize("M,G", [(2, 0), (8, 0), (3, 128), (16, 128)])
def test_w4a8_mfma_gemv_misaligned_x(M, G, off):
    """Activation rows that start 1 to 3 bytes past a 16-byte boundary take
    the MFMA GEMV's unaligned window loads; results stay bit-exact."""
    N, K = 50, 256
    c = WL.small_int_case(6000 + M + G + off, M, N, K, G)
    flat = dev(np.concatenate([np.zeros(off, np.int8), c["xq"].reshape(-1)]))
    xd = flat[off:].view(M, K)
    assert xd.data_ptr() % 16 == off
    y = q4.q4_linear_w4a8(xd, dev(c["sx"]), dev(c["w"]), dev(c["sw"]), G, "excess8")
    assert q4.q4_last_path() == "gemv"
    y_ref = L.linear_w4a8(c["xq"], c["sx"], c["w"], c["sw"], G, F.EXCESS8)
    assert_bitwise(host(y), y_ref, f"misaligned x +{off} M{M} G{G}")


@pytest.mark.parametrize("M", [20, 33])
def test_w4a16_mfma_gemv_misaligned_x(M):
    """bf16 activation rows 2 bytes past a 16-byte boundary on the W4A16
    MFMA GEMV (the route for 17 to 40 rows)."""
    N, K, G = 45, 512, 128
    c = WL.small_float_case(6100 + M, M, N, K, G)
    flat = dev(np.concatenate([np.zeros(1, np.uint16), c["x_bf16"].reshape(-1)]))
    xd = flat[1:].view(M, K)
    assert xd.data_ptr() % 16 != 0
    yb, yf = q4.q4_linear_w4a16(xd, dev(c["qweight"]), dev(c["scales_bf16"]), G, "excess8", want_f32=True)
    assert q4.q4_last_path() == "gemv"
    _w4a16_check(c, yb, yf, f"W4A16 misaligned x M{M}")


def test_w4a8_index_probe_through_gemv():
    """Codes that name their position, read back with one-hot activations."""
    N, K = 48, 256
    codes = ((np.arange(N)[:, None] * 3 + np.arange(K)[None, :] * 5) % 15) - 7
    xq = np.eye(K, dtype=np.int8)[:16]
    y = q4.q4_linear_w4a8(dev(xq), dev(np.ones(16, np.float32)), dev(F.pack_codes(codes, F.EXCESS8)),
                          dev(np.ones(N, np.float32)), 0, "excess8")
    assert_bitwise(host(y), codes.T[:16].astype(np.float32), "probe")


def test_w4a8_k_zero_and_empty():
    xq = dev(np.zeros((3, 0), np.int8))
    y = torch.full((3, 5), 7.0, device="cuda:0")
    q4.q4_linear_w4a8(xq, dev(np.ones(3, np.float32)), dev(np.zeros((5, 0), np.uint8)),
                      dev(np.ones(5, np.float32)), 0, "excess8", y=y)
    assert host(y).tolist() == [[0.0] * 5] * 3
    y0 = q4.q4_linear_w4a8(dev(np.zeros((0, 4), np.int8)), dev(np.zeros(0, np.float32)),
                           dev(np.zeros((5, 2), np.uint8)), dev(np.ones(5, np.float32)))
    assert tuple(y0.shape) == (0, 5)


@pytest.mark.parametrize("M,N,K,dt", [(1, 37, 32, "bf16"), (1, 70, 6144, "bf16"), (1, 21, 10240, "f32"),
                                      (2, 64, 2048, "f32"), (3, 40, 1000, "bf16"), (5, 33, 4095, "f32"),
                                      (8, 50, 2048, "bf16"), (16, 37, 2048, "bf16"), (16, 20, 1024, "f32")])
@pytest.mark.parametrize("enc", F.ENCODINGS)
@_paths("generic", "gemv", "auto")
def test_w4a8_dynamic_channel_decode_bitwise(M, N, K, dt, enc, path):
    """Per-channel dynamic W4A8 at decode sizes: the fused quantizer (one
    row on the default route, every row count on the forced decode route),
    float x, a zero row, odd K, several passes of K."""
    q4.q4_set_path(path)
    c = WL.small_int_case(M * 31 + N + K, M, N, K, 0)
    x = np.random.default_rng(M * 1000 + K).standard_normal((M, K), dtype=np.float32)
    if M > 1:
        x[1] = 0.0                      # scale 0, codes 0
    x[0, K // 3] = np.float32(-7.5)     # a row maximum that is negative
    xin = F.f32_to_bf16_bits(x) if dt == "bf16" else x
    y = q4.q4_linear_w4a8_dynamic(dev(xin), dev(c["w"]), dev(c["sw"]), 0, enc)
    y_ref, _, _ = L.linear_w4a8_dynamic(xin, c["w"], c["sw"], 0, enc, dt)
    assert_bitwise(host(y), y_ref, f"dynamic M{M} N{N} K{K} {dt} {enc} via {q4.q4_last_path()}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_w4a8_dynamic_channel_decode_extreme_rows(dt):
    """Rows whose maxima sit far outside the usual range (1e-30 .. 1e30,
    and a row with subnormal f32 values) take the plain division in the fused
    quantizer; the others the reciprocal form.  Codes must match the oracle's."""
    M, N, K = 6, 40, 2048
    c = WL.small_int_case(5150, M, N, K, 0)
    x = np.random.default_rng(99).standard_normal((M, K), dtype=np.float32)
    x[1] *= np.float32(1e-30)
    x[2] *= np.float32(1e30)
    x[3] *= np.float32(1e-19)
    x[4] *= np.float32(3e-40) if dt == "f32" else np.float32(1e-35)
    xin = F.f32_to_bf16_bits(x) if dt == "bf16" else x
    q4.q4_set_path("gemv")   # the fused quantizer serves every row count on this route
    y = q4.q4_linear_w4a8_dynamic(dev(xin), dev(c["w"]), dev(c["sw"]), 0, "excess8")
    assert q4.q4_last_path() == "gemv"
    y_ref, _, _ = L.linear_w4a8_dynamic(xin, c["w"], c["sw"], 0, F.EXCESS8, dt)
    assert_bitwise(host(y), y_ref, f"extreme rows {dt}")
    q4.q4_set_path("auto")
    for m in range(M):               # one row per call: the fused quantizer on the default route
        y1 = q4.q4_linear_w4a8_dynamic(dev(xin[m:m + 1]), dev(c["w"]), dev(c["sw"]), 0, "excess8")
        assert q4.q4_last_path() == "gemv"
        assert_bitwise(host(y1), y_ref[m:m + 1], f"extreme row {m} alone {dt}")


def test_w4a8_dynamic_channel_decode_misaligned_x():
    """A bf16 activation row that starts 2 bytes past a 16-byte boundary."""
    M, N, K = 2, 45, 2048
    c = WL.small_int_case(4242, M, N, K, 0)
    x = F.f32_to_bf16_bits(np.random.default_rng(7).standard_normal((M, K), dtype=np.float32))
    flat = dev(np.concatenate([np.zeros(1, np.uint16), x.reshape(-1)]))
    xd = flat[1:].view(M, K)
    assert xd.data_ptr() % 16 != 0
    y = q4.q4_linear_w4a8_dynamic(xd, dev(c["w"]), dev(c["sw"]), 0, "excess8")
    y_ref, _, _ = L.linear_w4a8_dynamic(x, c["w"], c["sw"], 0, F.EXCESS8, "bf16")
    assert_bitwise(host(y), y_ref, "misaligned x")


# (M, N, K, G, dt): activation matrices of at most 32 KB, which the default
# route quantizes inside the W4A8 MFMA GEMV (one launch, workspace unused)
FUSED_MFMA_CASES = [(4, 3072, 1023, 0, "f32"), (2, 96, 2048, 0, "f32"), (7, 70, 1023, 0, "bf16"),
                    (16, 50, 1024, 0, "bf16"), (20, 64, 768, 0, "bf16"), (3, 80, 2048, 128, "f32"),
                    (8, 45, 2048, 128, "bf16"), (12, 33, 1280, 256, "bf16"), (4, 40, 1536, 128, "f32"),
                    # whole units of four columns past K, and a partial one
                    (3, 64, 991, 0, "bf16"), (5, 40, 959, 0, "f32")]


@pytest.mark.parametrize("M,N,K,G,dt", FUSED_MFMA_CASES)
@pytest.mark.parametrize("enc", F.ENCODINGS)
def test_w4a8_dynamic_fused_mfma_bitwise(M, N, K, G, dt, enc):
    """The dynamic call with the quantizer inside the MFMA GEMV: outputs bit
    for bit the oracle's (quantize the rows, then W4A8), with a zero row, a
    negative row maximum, rows of tiny and huge magnitude (the plain-division
    codes), and the workspace left as it was (no separate quantizer ran)."""
    if G == 0 and enc == "twos":
        pytest.skip("per channel needs the biased pad")
    c = WL.small_int_case(M * 13 + N + K + G, M, N, K, G)
    x = np.random.default_rng(M * 77 + K).standard_normal((M, K), dtype=np.float32)
    x[0, K // 3] = np.float32(-9.25)
    if M > 1:
        x[1] = 0.0
    if M > 3:
        x[2] *= np.float32(1e-30)
        x[3] *= np.float32(1e30)
    xin = F.f32_to_bf16_bits(x) if dt == "bf16" else x
    ws = torch.full((q4.q4_w4a8_dynamic_workspace(M, K),), 0x5A, dtype=torch.uint8, device="cuda:0")
    y = q4.q4_linear_w4a8_dynamic(dev(xin), dev(c["w"]), dev(c["sw"]), G, enc, ws=ws)
    assert q4.q4_last_path() == "gemv"
    assert bool((ws == 0x5A).all()), "the workspace was written: the two-launch path ran"
    y_ref, _, _ = L.linear_w4a8_dynamic(xin, c["w"], c["sw"], G, enc, dt)
    assert_bitwise(host(y), y_ref, f"fused MFMA M{M} N{N} K{K} G{G} {dt} {enc}")
    # the same call through the library's own scratch array
    y2 = q4.q4_linear_w4a8_dynamic_noalloc(dev(xin), dev(c["w"]), dev(c["sw"]), G, enc)
    assert_bitwise(host(y2), y_ref, f"fused MFMA noalloc M{M} N{N} K{K} G{G} {dt} {enc}")


def test_w4a8_dynamic_fused_mfma_misaligned_x():
    """f32 and bf16 rows that start off a 16-byte boundary take the element
    loads of the fused quantizer."""
    M, N, K = 4, 64, 1024
    c = WL.small_int_case(8181, M, N, K, 0)
    x = np.random.default_rng(8).standard_normal((M, K), dtype=np.float32)
    for xin, pad in ((x, np.zeros(1, np.float32)), (F.f32_to_bf16_bits(x), np.zeros(1, np.uint16))):
        flat = dev(np.concatenate([pad, xin.reshape(-1)]))
        xd = flat[1:].view(M, K)
        assert xd.data_ptr() % 16 != 0
        y = q4.q4_linear_w4a8_dynamic(xd, dev(c["w"]), dev(c["sw"]), 0, "excess8")
        y_ref, _, _ = L.linear_w4a8_dynamic(xin, c["w"], c["sw"], 0, F.EXCESS8,
                                            "bf16" if xin.dtype == np.uint16 else "f32")
        assert_bitwise(host(y), y_ref, f"fused misaligned {xin.dtype}")


def test_microdecoder_linears_bitwise():
    """Three of the stack's shapes (2048x2048, 5632x2048, 2048x5632) at M=1."""
    for idx in (0, 4, 6):
        d = WL.microdecoder_linear(idx)
        packed, sw = q4.q4_quantize_matrix(d["W"])
        p_ref, sw_ref = Q.quantize_q4_matrix(d["W"])
        assert_bitwise(packed, p_ref, "packed")
        y = q4.q4_linear_w4a8_dynamic(dev(d["x"]), dev(packed), dev(sw), 0, "excess8")
        y_ref, _, _ = L.linear_w4a8_dynamic(d["x"], p_ref, sw_ref, 0, F.EXCESS8, "bf16")
        assert_bitwise(host(y), y_ref, f"linear {idx}")


# --------------------------------------------------------------------------
# several per-channel linears in one launch (q4_linear_w4a8_dynamic_multi)
# --------------------------------------------------------------------------

MULTI_SHAPES = [(37, 32), (70, 6144), (1, 1023), (16, 2048), (2048, 2048), (21, 10240), (33, 4095), (0, 64),
                (40, 0), (5, 8160)]


def _multi_case(M, dt, shapes, seed):
    cases = []
    for i, (N, K) in enumerate(shapes):
        c = WL.small_int_case(seed + 17 * i, M, N, K, 0)
        x = np.random.default_rng(seed + i).standard_normal((M, K), dtype=np.float32)
        if M > 1 and K > 0:
            x[1] = 0.0                          # scale 0, codes 0
        if K > 0:
            x[0, K // 3] = np.float32(-7.5)     # a row maximum that is negative
        cases.append((F.f32_to_bf16_bits(x) if dt == "bf16" else x, c["w"], c["sw"]))
    return cases


@pytest.mark.parametrize("M,dt", [(1, "bf16"), (1, "f32"), (2, "bf16"), (5, "f32"), (16, "bf16")])
def test_w4a8_dynamic_multi_bitwise(M, dt):
    """Ten problems of different N and K (ragged N, odd K, several passes,
    N == 0, K == 0) in one launch: every output equals the oracle's and the
    single call's, bit for bit."""
    mp = 1 << (M - 1).bit_length()
    # the activation codes of one workgroup fit in 64 KB of LDS
    shapes = [(N, K) for N, K in MULTI_SHAPES if mp * -(-K // 2048) <= 31]
    cases = _multi_case(M, dt, shapes, 300 + M)
    ys = q4.q4_linear_w4a8_dynamic_multi([(dev(x), dev(w), dev(sw)) for x, w, sw in cases])
    assert q4.q4_last_path() == "gemv"
    q4.q4_set_path("gemv")
    for (x, w, sw), y in zip(cases, ys):
        N, K = w.shape[0], x.shape[1]
        y_ref, _, _ = L.linear_w4a8_dynamic(x, w, sw, 0, F.EXCESS8, dt)
        assert_bitwise(host(y), y_ref, f"multi M{M} N{N} K{K} {dt}")
        if N and K:
            y1 = q4.q4_linear_w4a8_dynamic(dev(x), dev(w), dev(sw), 0, "excess8")
            assert_bitwise(host(y1), host(y), f"multi vs single M{M} N{N} K{K}")


def test_w4a8_dynamic_multi_sixty_four_problems():
    """The most problems one launch takes, each a few rows."""
    shapes = [(1 + (i * 7) % 40, 32 * (1 + i % 5)) for i in range(q4.MULTI_MAX)]
    cases = _multi_case(1, "bf16", shapes, 900)
    ys = q4.q4_linear_w4a8_dynamic_multi([(dev(x), dev(w), dev(sw)) for x, w, sw in cases])
    for i, ((x, w, sw), y) in enumerate(zip(cases, ys)):
        y_ref, _, _ = L.linear_w4a8_dynamic(x, w, sw, 0, F.EXCESS8, "bf16")
        assert_bitwise(host(y), y_ref, f"problem {i}")


@pytest.mark.parametrize("M,dt", [(1, "bf16"), (4, "f32")])
def test_w4a8_dynamic_multi_two_tiles_per_workgroup(M, dt):
    """A launch of more than 4096 tiles of 16 rows, where each workgroup
    takes two consecutive tiles: ragged problems end on a one-tile
    workgroup, and every row is written once with the oracle's value."""
    shapes = [(70, 6144), (65536 + 16, 64), (37, 1023), (33, 4095), (16, 2048), (1, 32)]
    cases = _multi_case(M, dt, shapes, 4242 + M)
    ys = q4.q4_linear_w4a8_dynamic_multi([(dev(x), dev(w), dev(sw)) for x, w, sw in cases])
    for i, ((x, w, sw), y) in enumerate(zip(cases, ys)):
        y_ref, _, _ = L.linear_w4a8_dynamic(x, w, sw, 0, F.EXCESS8, dt)
        assert_bitwise(host(y), y_ref, f"two tiles: M{M} problem {i} N{w.shape[0]} K{x.shape[1]}")


def test_w4a8_dynamic_multi_shared_input():
    """q, k and v style: three problems read the same activation tensor (a
    shared input is allowed; only outputs may not overlap anything)."""
    K = 2048
    x = np.random.default_rng(31).standard_normal((1, K), dtype=np.float32)
    xb = F.f32_to_bf16_bits(x)
    xd = dev(xb)
    cases = [WL.small_int_case(3100 + i, 1, N, K, 0) for i, N in enumerate((2048, 512, 512))]
    ys = q4.q4_linear_w4a8_dynamic_multi([(xd, dev(c["w"]), dev(c["sw"])) for c in cases])
    for i, (c, y) in enumerate(zip(cases, ys)):
        y_ref, _, _ = L.linear_w4a8_dynamic(xb, c["w"], c["sw"], 0, F.EXCESS8, "bf16")
        assert_bitwise(host(y), y_ref, f"shared input, problem {i}")


def test_w4a8_dynamic_multi_microdecoder_pass():
    """One pass of the microdecoder stack (35 linears: 2048x2048, 5632x2048,
    2048x5632) in one launch, each output against the oracle."""
    lin = WL.microdecoder_linears()
    cases = []
    for i in range(len(lin)):
        d = WL.microdecoder_linear(i)
        packed, sw = q4.q4_quantize_matrix(d["W"])   # pinned to the oracle's quantizer on the host
        cases.append((d["x"], packed, sw))
    ys = q4.q4_linear_w4a8_dynamic_multi([(dev(x), dev(w), dev(sw)) for x, w, sw in cases])
    for i, ((x, w, sw), y) in enumerate(zip(cases, ys)):
        y_ref, _, _ = L.linear_w4a8_dynamic(x, w, sw, 0, F.EXCESS8, "bf16")
        assert_bitwise(host(y), y_ref, f"microdecoder linear {i} {lin[i][1]}")


def test_w4a8_dynamic_multi_graph_replays():
    """Captured in a HIP graph and replayed three times, with eager work and
    synchronisation between replays: every replay equals the eager result."""
    cases = _multi_case(1, "bf16", [(70, 6144), (2048, 2048), (37, 0), (33, 4095)], 1234)
    probs = [(dev(x), dev(w), dev(sw)) for x, w, sw in cases]
    eager = [host(y).copy() for y in q4.q4_linear_w4a8_dynamic_multi(probs)]
    ys = [torch.full((1, w.shape[0]), float("nan"), dtype=torch.float32, device="cuda:0") for _, w, _ in cases]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q4.q4_linear_w4a8_dynamic_multi(probs, ys=ys)
    for r in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            assert_bitwise(host(y), eager[i], f"replay {r} problem {i}")
        q4.q4_linear_w4a8_dynamic_multi(probs)      # eager work between replays


# The prefill workload (M=2048, N=13312, K=2048, G=128) is compared on every
# output element.  The routed call runs once per process (cached); the oracle
# then takes the rows in blocks of 512, since rows are independent in its
# definition, which keeps its integer accumulators near 1 GB per block.
PREFILL_BLOCKS = [(r, r + 512) for r in range(0, 2048, 512)]


@functools.lru_cache(maxsize=1)
def _prefill_w4a8_run():
    q4.q4_set_path("auto")
    d = WL.w4a8_prefill()
    y = q4.q4_linear_w4a8_dynamic(dev(d["x"]), dev(d["qweight"]), dev(d["scales"]), 128, "excess8")
    path = q4.q4_last_path()
    xq_ref, sx_ref = Q.quantize_q8_rows(d["x"], "bf16")
    return d, host(y), path, xq_ref, sx_ref


@pytest.mark.parametrize("r0,r1", PREFILL_BLOCKS)
def test_w4a8_prefill_full_size_every_element(r0, r1):
    """The dynamic grouped W4A8 call at the prefill workload through the
    default (tiled) route: rows r0..r1 of y bit for bit against the oracle
    (quantize the bf16 rows, then the grouped linear)."""
    d, yh, path, xq_ref, sx_ref = _prefill_w4a8_run()
    assert path == "tiled"
    y_ref = L.linear_w4a8(xq_ref[r0:r1], sx_ref[r0:r1], d["qweight"], d["scales"], 128, F.EXCESS8)
    assert_bitwise(yh[r0:r1], y_ref, f"prefill rows {r0}..{r1} via {path}")


# The tiled W4A8 kernel splits the tiles past its last whole round of
# workgroups (two per CU, 512 on MI355X's 256 CUs) into quarter tiles when
# they fill at most a quarter of a round, into halves up to half a round.
# 576 tiles (8 columns of tiles x 72 rows) leave 64 for quarters, 712 leave
# 200 for halves; both shapes are ragged in M and N.
@pytest.mark.parametrize("M,N,G", [(72 * 128 - 5, 1000, 128), (89 * 128 - 7, 1024, 128),
                                   (72 * 128 - 5, 1000, 0), (89 * 128 - 7, 1024, 0)])
def test_w4a8_tiled_tail_split_every_element(M, N, G):
    c = WL.small_int_case(M + N + G, M, N, 256, G)
    y = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), G, "excess8")
    assert q4.q4_last_path() == "tiled"
    y_ref = L.linear_w4a8(c["xq"], c["sx"], c["w"], c["sw"], G, F.EXCESS8)
    assert_bitwise(host(y), y_ref, f"tail split M{M} N{N} G{G}")


# --------------------------------------------------------------------------
# float activations (tolerance against the float64 oracle)
# --------------------------------------------------------------------------

def _w4a16_check(c, yb, yf, what):
    _w4a16_check_host(c, host(yb), host(yf), what)


def _w4a16_check_host(c, yb_h, yf_h, what):
    x64 = F.bf16_bits_to_f32(c["x_bf16"] if "x_bf16" in c else c["x"]).astype(np.float64)
    s64 = F.bf16_bits_to_f32(c["scales_bf16"]).astype(np.float64)
    y_ref = L.linear_w4a16(c["x_bf16"] if "x_bf16" in c else c["x"], c["qweight"], c["scales_bf16"],
                           c["G"], c["enc"])
    terms = L.abs_terms(x64, c["qweight"], s64, c["K"], c["G"], c["enc"])
    assert_close(yf_h, y_ref, terms, F32_TOL, what + " f32")
    assert_close(F.bf16_bits_to_f32(yb_h), y_ref, terms, BF16_TOL, what + " bf16")
    assert_bitwise(yb_h, F.f32_to_bf16_bits(yf_h), what + " bf16 = rne(f32)")


@pytest.mark.parametrize("M,N,K,G", [(1, 37, 256, 128), (4, 80, 384, 128), (8, 128, 1024, 256),
                                     (16, 45, 512, 128), (17, 64, 256, 128), (3, 40, 384, 32),
                                     (2, 37, 384, 2), (5, 33, 384, 64), (16, 64, 2048, 128),
                                     (13, 40, 4096, 256),
                                     # decode: several 2048-wide passes, a ragged last pass
                                     (1, 70, 5632, 128), (2, 33, 10240, 64), (7, 20, 6144, 32),
                                     (12, 19, 4608, 128), (5, 50, 4096, 512), (2, 30, 8192, 4096),
                                     (6, 24, 6144, 384), (9, 70, 2048, 2048), (3, 33, 8192, 128),
                                     (1, 20, 10240, 256),
                                     # tiled: ragged tiles, G spanning 1, 2 and 4 K steps
                                     (40, 96, 512, 128), (130, 200, 1024, 64), (129, 129, 256, 256),
                                     (64, 130, 2048, 128),
                                     # tiled: one K step, two, three (one turn of the staging ring)
                                     (33, 64, 64, 64), (40, 50, 128, 128), (20, 256, 192, 64),
                                     # tiled in 64-row halves: every tile (at most 64 rows, XCD
                                     # remap), the tiles past the last whole round of workgroups
                                     (48, 1024, 384, 128), (130, 36864, 256, 128)])
@pytest.mark.parametrize("enc", F.ENCODINGS)
@_paths("generic", "gemv", "gemv_mc", "tiled", "auto")
def test_w4a16_tolerance(M, N, K, G, enc, path):
    q4.q4_set_path(path)
    c = WL.small_float_case(M * 13 + N + K + G, M, N, K, G, enc)
    yb, yf = q4.q4_linear_w4a16(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), G, enc,
                                want_f32=True)
    _w4a16_check(c, yb, yf, f"W4A16 M{M} N{N} K{K} G{G} {enc} via {q4.q4_last_path()}")


@pytest.mark.parametrize("M", [1, 4, 8])
@_paths("auto", "gemv_mc")
def test_w4a16_decode_workload(M, path):
    """N=13312, K=2048, G=128 at M in {1, 4, 8}, full size."""
    q4.q4_set_path(path)
    d = WL.w4a16_gemv()
    c = dict(x_bf16=d["x"][M], qweight=d["qweight"], scales_bf16=d["scales_bf16"], G=128,
             enc="excess8", K=2048)
    yb, yf = q4.q4_linear_w4a16(dev(c["x_bf16"]), dev(d["qweight"]), dev(d["scales_bf16"]), 128, "excess8",
                                want_f32=True)
    _w4a16_check(c, yb, yf, f"decode M{M} via {q4.q4_last_path()}")


@pytest.mark.parametrize("N,K", ROUTE_SHAPES)
def test_w4a16_route_by_batch(N, K):
    """The default W4A16 route follows the measured plan: the streaming
    decode kernel for M <= 16 on every shape, the MFMA GEMV up to the
    shape's crossing, tiled above; sampled columns against the oracle."""
    dmax = q4.q4_route_plan("w4a16", 1, N, K, 128)["decode_max"]
    assert dmax >= 16
    cols = _route_cols(N)
    for M in _route_ms(dmax):
        want = "gemv" if M <= dmax else "tiled"
        assert q4.q4_route_plan("w4a16", M, N, K, 128)["path"] == want, (M, N, K)
        c = WL.small_float_case(M + N + K, M, N, K, 128)
        yb, yf = q4.q4_linear_w4a16(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), 128, "excess8",
                                    want_f32=True)
        assert q4.q4_last_path() == want, (M, N, K)
        cs = dict(c, qweight=c["qweight"][cols], scales_bf16=c["scales_bf16"][cols], N=len(cols))
        _w4a16_check_host(cs, host(yb)[:, cols], host(yf)[:, cols], f"route M{M} N{N} K{K} via {want}")


@functools.lru_cache(maxsize=1)
def _prefill_w4a16_run():
    q4.q4_set_path("auto")
    d = WL.w4a16_gemv(Ms=(1,))
    x = WL.w4a8_prefill()["x"]                      # bf16 bits [2048, 2048]
    yb, yf = q4.q4_linear_w4a16(dev(x), dev(d["qweight"]), dev(d["scales_bf16"]), 128, "excess8",
                                want_f32=True)
    return d, x, host(yb), host(yf), q4.q4_last_path()


@pytest.mark.parametrize("r0,r1", PREFILL_BLOCKS)
def test_w4a16_prefill_shape_every_element(r0, r1):
    """The prefill shape with W4A16 types (x bf16 [2048, 2048], packed
    [13312, 1024], bf16 scales [13312, 16], G=128) through the tiled kernel:
    rows r0..r1 against the float64 oracle, normwise over the block and
    conditioned per element, and bf16 = RNE(f32) bit for bit."""
    d, x, yb, yf, path = _prefill_w4a16_run()
    assert path == "tiled"
    c = dict(x_bf16=x[r0:r1], qweight=d["qweight"], scales_bf16=d["scales_bf16"], G=128, enc="excess8", K=2048)
    _w4a16_check_host(c, yb[r0:r1], yf[r0:r1], f"prefill-shape W4A16 rows {r0}..{r1}")


def test_w4a16_batch_invariance():
    """A row's bits do not depend on the batch it is computed in (decode path)."""
    d = WL.w4a16_gemv()
    x8 = d["x"][8]
    w, s = dev(d["qweight"]), dev(d["scales_bf16"])
    _, y8 = q4.q4_linear_w4a16(dev(x8), w, s, 128, "excess8", want_f32=True)
    y8h = host(y8)
    for m in range(8):
        _, y1 = q4.q4_linear_w4a16(dev(x8[m:m + 1]), w, s, 128, "excess8", want_f32=True)
        assert_bitwise(host(y1)[0], y8h[m], f"row {m}")
    _, y8b = q4.q4_linear_w4a16(dev(x8), w, s, 128, "excess8", want_f32=True)
    assert_bitwise(host(y8b), y8h, "repeat")


@pytest.mark.parametrize("enc", F.ENCODINGS)
@pytest.mark.parametrize("path,G", [("auto", 128), ("auto", 64), ("gemv_mc", 128), ("gemv_mc", 512)])
def test_w4a16_batch_invariance_every_m(enc, path, G):
    """Rows of a 16-row batch equal those of every smaller batch, bit for bit,
    over several chunks of K with a ragged last one."""
    q4.q4_set_path(path)
    c = WL.small_float_case(977, 16, 100, 5632 if G != 512 else 5120, G, enc)
    x, w, s = dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"])
    _, y16 = q4.q4_linear_w4a16(x, w, s, G, enc, want_f32=True)
    assert q4.q4_last_path() == ("gemv" if path == "auto" else path)
    y16h = host(y16)
    for m in range(1, 16):
        _, ym = q4.q4_linear_w4a16(x[:m].contiguous(), w, s, G, enc, want_f32=True)
        assert_bitwise(host(ym), y16h[:m], f"M={m}")


def _zero_code_case(seed, M, enc, zero_rows, N=96, K=4096, G=128):
    """A float case whose weight rows zero_rows hold only the code 0 (the
    stored byte 0x88 in excess-8 form, 0x00 in two's complement)."""
    c = WL.small_float_case(seed, M, N, K, G, enc)
    q = c["qweight"].copy()
    q[list(zero_rows)] = 0x88 if enc == F.EXCESS8 else 0x00
    return dict(c, qweight=q)


ZERO_ROWS = (0, 5, 17, 63, 95)


@pytest.mark.parametrize("enc", F.ENCODINGS)
@pytest.mark.parametrize("M", [1, 4, 16])
def test_w4a16_zero_code_rows_exact_on_decode(enc, M):
    """A weight row of zero codes gives exactly y = 0 on the default decode
    route, as its dequantized row does (the fused result equals
    dequantize-then-matmul, "Fused int4 and int8 dequantize-matmul in C",
    What the tests check); the conditioned check below demands an exact 0
    wherever the sum of |x q s| is 0, and tolerance elsewhere."""
    q4.q4_set_path("auto")
    c = _zero_code_case(4242 + M, M, enc, ZERO_ROWS)
    yb, yf = q4.q4_linear_w4a16(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), 128, enc,
                                want_f32=True)
    assert q4.q4_last_path() == "gemv"
    yfh, ybh = host(yf), host(yb)
    assert np.all(yfh[:, list(ZERO_ROWS)] == 0.0) and np.all(ybh[:, list(ZERO_ROWS)] == 0)
    _w4a16_check_host(c, ybh, yfh, f"zero-code rows M{M} {enc}")


@pytest.mark.parametrize("path,M,zp", [("gemv_mc", 4, False), ("gemv_mc", 16, False), ("tiled", 40, False),
                                       ("generic", 3, False), ("auto", 24, False), ("auto", 1, True),
                                       ("auto", 40, True)])
def test_w4a16_zero_code_rows_residue(path, M, zp):
    """The other W4A16 routes (and every route with zero points, for rows of
    codes equal to their zero point) subtract the bias term in rounded
    arithmetic: such a row may leave a residue instead of an exact 0.  It
    stays below the f32 tolerance times the size of the bias term,
    16 sum_g s_g (1 + z_g/16) sum_{k in g} |x_k|; the other rows pass the
    usual checks."""
    q4.q4_set_path(path)
    enc = F.EXCESS8
    c = _zero_code_case(777 + M, M, enc, ZERO_ROWS)
    G, K = c["G"], c["K"]
    x = F.bf16_bits_to_f32(c["x_bf16"]).astype(np.float64)
    s = F.bf16_bits_to_f32(c["scales_bf16"]).astype(np.float64)
    if zp:
        rng = np.random.default_rng(31 + M)
        z = rng.integers(0, 16, (c["N"], K // G)).astype(np.uint8)
        # rows of ZERO_ROWS hold, in each group, the group's zero point
        q = c["qweight"].copy()
        for r in ZERO_ROWS:
            u = np.repeat(z[r], G).astype(np.uint8)
            q[r] = u[0::2] | (u[1::2] << 4)
        yb, yf = q4.q4_linear_w4a16_zp(dev(c["x_bf16"]), dev(q), dev(c["scales_bf16"]), dev(z), G,
                                       want_f32=True)
        bias = 1.0 + z.astype(np.float64) / 16.0
    else:
        yb, yf = q4.q4_linear_w4a16(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), G, enc,
                                    want_f32=True)
        bias = np.full((c["N"], K // G), 1.5)
    yfh = host(yf)
    xg = np.abs(x).reshape(M, K // G, G).sum(axis=2)                 # [M, groups]
    for r in ZERO_ROWS:
        size = 16.0 * (xg * (s[r] * bias[r])[None, :]).sum(axis=1)   # [M]
        assert np.all(np.abs(yfh[:, r]) <= F32_TOL * size), (path, M, zp, r, np.abs(yfh[:, r]).max())
    live = [n for n in range(c["N"]) if n not in ZERO_ROWS]
    if not zp:
        cs = dict(c, qweight=c["qweight"][live], scales_bf16=c["scales_bf16"][live], N=len(live))
        _w4a16_check_host(cs, host(yb)[:, live], yfh[:, live], f"zero-code residue {path} M{M}")


@pytest.mark.parametrize("M,N,K,G", [(1, 2048, 2048, 32), (3, 37, 384, 2), (16, 64, 256, 64),
                                     (20, 40, 128, 128), (1, 37, 96, 32), (2, 33, 4096, 64), (5, 70, 2080, 32),
                                     (1, 13, 6144, 128), (7, 1, 2048, 2048), (1, 8200, 64, 32)])
@pytest.mark.parametrize("enc", F.ENCODINGS)
@_paths("generic", "gemv", "auto")
def test_w4a32_tolerance(M, N, K, G, enc, path):
    q4.q4_set_path(path)
    if (M, N, K) == (1, 2048, 2048):
        d = WL.w4a32_gemv()
        x, w, s = d["x"], d["qweight"], d["scales_f16"]
    else:
        c = WL.small_float_case(M + N + K + G, M, N, K, G, enc)
        x, w, s = c["x_f32"], c["qweight"], c["scales_f16"]
    y = q4.q4_linear_w4a32(dev(x), dev(w), dev(s, torch.float16), G, enc)
    y_ref = L.linear_w4a32(x, w, s, G, enc)
    terms = L.abs_terms(x.astype(np.float64), w, F.f16_bits_to_float(s), K, G, enc)
    assert_close(host(y), y_ref, terms, F32_TOL, f"W4A32 M{M} N{N} K{K} G{G} {enc}")


def test_w4a32_batch_invariance():
    """Each row of a 5-row W4A32 call equals the same row alone, bit for bit."""
    M, N, K, G = 5, 70, 4096, 32
    c = WL.small_float_case(777, M, N, K, G, "twos")
    w, s = dev(c["qweight"]), dev(c["scales_f16"], torch.float16)
    y = host(q4.q4_linear_w4a32(dev(c["x_f32"]), w, s, G, "twos"))
    assert q4.q4_last_path() == "gemv"
    for m in range(M):
        y1 = host(q4.q4_linear_w4a32(dev(c["x_f32"][m:m + 1]), w, s, G, "twos"))
        assert_bitwise(y1, y[m:m + 1], f"W4A32 row {m}")


def test_w4a32_f16_subnormal_scale():
    """f16 scale 0x0001 = 2^-24 must survive (no denormal flushing)."""
    codes = np.full((1, 4), 7)
    y = q4.q4_linear_w4a32(dev(np.ones((1, 4), np.float32)), dev(F.pack_codes(codes, F.TWOS)),
                           dev(np.array([[0x0001, 0x3555]], np.uint16), torch.float16), 2)
    want = 14.0 * 2.0 ** -24 + 14.0 * 0.333251953125
    assert abs(host(y)[0, 0] - want) <= 1e-6 * want
    # the same scales on the streaming kernel (groups of 32)
    codes = np.full((1, 64), 7)
    y = q4.q4_linear_w4a32(dev(np.ones((1, 64), np.float32)), dev(F.pack_codes(codes, F.TWOS)),
                           dev(np.array([[0x0001, 0x3555]], np.uint16), torch.float16), 32)
    assert q4.q4_last_path() == "gemv"
    want = 224.0 * 2.0 ** -24 + 224.0 * 0.333251953125
    assert abs(host(y)[0, 0] - want) <= 1e-6 * want


def test_float_k_zero():
    yb, yf = q4.q4_linear_w4a16(dev(np.zeros((2, 0), np.uint16)), dev(np.zeros((3, 0), np.uint8)),
                                dev(np.zeros((3, 0), np.uint16)), 2, "excess8", want_f32=True)
    assert host(yf).tolist() == [[0.0] * 3] * 2 and host(yb).tolist() == [[0] * 3] * 2


# --------------------------------------------------------------------------
# per-group zero points ("The 4-bit CPU path", section W4A8)
# --------------------------------------------------------------------------

def _zeros(seed, N, Gn):
    return np.random.default_rng(seed).integers(0, 16, (N, Gn)).astype(np.uint8)


ZP_W4A16_CASES = [  # M, N, K, G: decode (streaming), MFMA GEMV rows, tiled with ragged tiles
    (1, 37, 256, 128), (4, 80, 2048, 128), (16, 45, 512, 64), (1, 64, 4096, 256),
    (24, 64, 1024, 128), (40, 33, 2048, 128), (130, 200, 1024, 128), (64, 96, 512, 256),
    (40, 1024, 512, 128), (130, 36864, 256, 128)]


@pytest.mark.parametrize("M,N,K,G", ZP_W4A16_CASES)
@_paths("generic", "gemv", "tiled", "auto")
def test_w4a16_zero_points_tolerance(M, N, K, G, path):
    q4.q4_set_path(path)
    c = WL.small_float_case(M * 13 + N + K + G, M, N, K, G)
    z = _zeros(M + N + K, N, K // G)
    yb, yf = q4.q4_linear_w4a16_zp(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), dev(z), G,
                                   want_f32=True)
    y_ref = L.linear_w4a16_zp(c["x_bf16"], c["qweight"], c["scales_bf16"], z, G)
    x64 = F.bf16_bits_to_f32(c["x_bf16"]).astype(np.float64)
    codes = np.abs(L.codes_with_zero_points(c["qweight"], z, K, G)).astype(np.float64)
    s64 = F.bf16_bits_to_f32(c["scales_bf16"]).astype(np.float64)
    terms = np.zeros((M, N))
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        terms += (np.abs(x64[:, ks]) @ codes[:, ks].T) * s64[None, :, g]
    what = f"W4A16 zp M{M} N{N} K{K} G{G} via {q4.q4_last_path()}"
    yf_h, yb_h = host(yf), host(yb)
    assert_close(yf_h, y_ref, terms, F32_TOL, what + " f32")
    assert_close(F.bf16_bits_to_f32(yb_h), y_ref, terms, BF16_TOL, what + " bf16")
    assert_bitwise(yb_h, F.f32_to_bf16_bits(yf_h), what + " bf16 = rne(f32)")


@pytest.mark.parametrize("M", [1, 4, 24])
@_paths("generic", "gemv", "auto")
def test_w4a16_zero_point_8_is_symmetric(M, path):
    """z = 8 everywhere on the decode and generic routes: the same bits as
    the symmetric excess-8 call (the correction constant is exactly -1.5)."""
    q4.q4_set_path(path)
    N, K, G = 70, 2048, 128
    c = WL.small_float_case(M + 77, M, N, K, G)
    z8 = np.full((N, K // G), 8, np.uint8)
    yb, yf = q4.q4_linear_w4a16_zp(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), dev(z8), G,
                                   want_f32=True)
    yb2, yf2 = q4.q4_linear_w4a16(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), G, "excess8",
                                  want_f32=True)
    assert_bitwise(host(yf), host(yf2), f"z=8 vs symmetric M{M} via {q4.q4_last_path()}")


def test_w4a16_zero_points_batch_invariance():
    """Decode rows with zero points: a row's bits are the same alone and in a
    batch of 16 (one streaming kernel for every M <= 16)."""
    N, K, G = 96, 2048, 128
    c = WL.small_float_case(4321, 16, N, K, G)
    z = _zeros(99, N, K // G)
    _, y16 = q4.q4_linear_w4a16_zp(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), dev(z), G,
                                   want_f32=True)
    y16 = host(y16)
    for m in (0, 5, 15):
        _, y1 = q4.q4_linear_w4a16_zp(dev(c["x_bf16"][m:m + 1]), dev(c["qweight"]), dev(c["scales_bf16"]),
                                      dev(z), G, want_f32=True)
        assert_bitwise(host(y1), y16[m:m + 1], f"row {m}")


ZP_W4A8_CASES = [  # M, N, K, G
    (1, 37, 256, 128), (5, 80, 2048, 128), (16, 45, 1024, 256), (17, 64, 512, 128), (40, 33, 2048, 128),
    (130, 70, 1024, 128), (6, 37, 384, 2), (3, 40, 384, 64), (9, 40, 5632, 128)]


@pytest.mark.parametrize("M,N,K,G", ZP_W4A8_CASES)
@_paths("generic", "gemv", "tiled", "auto")
def test_w4a8_zero_points_bitwise(M, N, K, G, path):
    q4.q4_set_path(path)
    c = WL.small_int_case(M * 11 + N + K + G, M, N, K, G)
    z = _zeros(M * 3 + K, N, K // G)
    y = q4.q4_linear_w4a8_zp(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), dev(z), G)
    y_ref = L.linear_w4a8_zp(c["xq"], c["sx"], c["w"], c["sw"], z, G)
    assert_bitwise(host(y), y_ref, f"W4A8 zp M{M} N{N} K{K} G{G} via {q4.q4_last_path()}")


def test_w4a8_zero_point_8_is_symmetric():
    """z = 8 everywhere: bit for bit the symmetric excess-8 grouped result,
    on the decode route and at a prefill size (tiled vs MFMA GEMV)."""
    for M in (3, 300):
        N, K, G = 96, 1024, 128
        c = WL.small_int_case(M + 5, M, N, K, G)
        z8 = np.full((N, K // G), 8, np.uint8)
        y = q4.q4_linear_w4a8_zp(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), dev(z8), G)
        y2 = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), G, "excess8")
        assert_bitwise(host(y), host(y2), f"z=8 M{M}")


def test_w4a8_zero_points_extreme():
    """xq = +-127 against u = 15, z = 0 (the largest |u - z|): the exact
    closed form 127 * 15 * K per output."""
    M, N, K, G = 2, 16, 2048, 128
    xq = np.full((M, K), 127, np.int8)
    xq[1] = -127
    w = np.full((N, K // 2), 0xFF, np.uint8)
    z = np.zeros((N, K // G), np.uint8)
    one = np.ones(M, np.float32)
    y = q4.q4_linear_w4a8_zp(dev(xq), dev(one), dev(w), dev(np.ones((N, K // G), np.float32)), dev(z), G)
    assert_bitwise(host(y), np.array([[127.0 * 15 * K] * N, [-127.0 * 15 * K] * N], np.float32), "extreme zp")


@functools.lru_cache(maxsize=1)
def _prefill_zp_run():
    q4.q4_set_path("auto")
    d = WL.w4a8_prefill()
    xq, sx = Q.quantize_q8_rows(d["x"], "bf16")
    z = _zeros(2024, d["N"], d["K"] // 128)
    y = q4.q4_linear_w4a8_zp(dev(xq), dev(sx), dev(d["qweight"]), dev(d["scales"]), dev(z), 128)
    return d, xq, sx, z, host(y), q4.q4_last_path()


@pytest.mark.parametrize("r0,r1", PREFILL_BLOCKS)
def test_w4a8_zero_points_prefill_full_size_every_element(r0, r1):
    """M=2048, N=13312, K=2048, G=128 with random zero points through the
    routed (tiled) kernel: rows r0..r1 bit for bit."""
    d, xq, sx, z, yh, path = _prefill_zp_run()
    assert path == "tiled"
    y_ref = L.linear_w4a8_zp(xq[r0:r1], sx[r0:r1], d["qweight"], d["scales"], z, 128)
    assert_bitwise(yh[r0:r1], y_ref, f"zp prefill rows {r0}..{r1}")


# --------------------------------------------------------------------------
# int8 weights, one scale per row, float activations (W8A32, W8A16)
# --------------------------------------------------------------------------

def _w8_case(seed, M, N, K):
    rng = np.random.default_rng(seed)
    wq = rng.integers(-128, 128, (N, K)).astype(np.int8)
    wq[0, :min(K, 3)] = -128                             # the most negative code
    sw = rng.uniform(0.001, 0.05, N).astype(np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    return wq, sw, x


def _w8_terms(x64, wq, sw):
    return (np.abs(x64) @ np.abs(wq.astype(np.float64)).T) * np.abs(sw.astype(np.float64))[None, :]


@_paths("generic", "gemv", "auto")
def test_w8_worked_example(path):
    """The int8 form of the worked example: [-13, 5] exactly, f32 and bf16 x."""
    q4.q4_set_path(path)
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
    wq = np.array(g["codes"], np.int8)
    sw = np.array(g["int8_row_scales"], np.float32)
    x = np.array([g["x"]], np.float32)
    y = q4.q8_linear_w8a32(dev(x), dev(wq), dev(sw))
    assert host(y).tolist() == [g["int8_y"]]
    yb, yf = q4.q8_linear_w8a16(dev(F.f32_to_bf16_bits(x)), dev(wq), dev(sw), want_f32=True)
    assert host(yf).tolist() == [g["int8_y"]]
    assert F.bf16_bits_to_f32(host(yb)).tolist() == [g["int8_y"]]


W8_CASES = [(1, 37, 256), (2, 64, 2048), (3, 40, 1040), (4, 80, 4096), (16, 33, 1024), (17, 45, 512),
            (40, 70, 2048), (130, 96, 256), (5, 19, 8), (2, 21, 1000)]   # last two: K % 16 != 0 (generic)


@pytest.mark.parametrize("M,N,K", W8_CASES)
@_paths("generic", "gemv", "auto")
def test_w8a32_tolerance(M, N, K, path):
    q4.q4_set_path(path)
    wq, sw, x = _w8_case(M * 7 + N + K, M, N, K)
    y = q4.q8_linear_w8a32(dev(x), dev(wq), dev(sw))
    y_ref = L.linear_w8a32(x, wq, sw)
    assert_close(host(y), y_ref, _w8_terms(x.astype(np.float64), wq, sw), F32_TOL,
                 f"W8A32 M{M} N{N} K{K} via {q4.q4_last_path()}")


@pytest.mark.parametrize("M,N,K", W8_CASES)
@_paths("generic", "gemv", "auto")
def test_w8a16_tolerance(M, N, K, path):
    q4.q4_set_path(path)
    wq, sw, x = _w8_case(M * 5 + N + K, M, N, K)
    xb = F.f32_to_bf16_bits(x)
    yb, yf = q4.q8_linear_w8a16(dev(xb), dev(wq), dev(sw), want_f32=True)
    y_ref = L.linear_w8a16(xb, wq, sw)
    terms = _w8_terms(F.bf16_bits_to_f32(xb).astype(np.float64), wq, sw)
    what = f"W8A16 M{M} N{N} K{K} via {q4.q4_last_path()}"
    yf_h, yb_h = host(yf), host(yb)
    assert_close(yf_h, y_ref, terms, F32_TOL, what + " f32")
    assert_close(F.bf16_bits_to_f32(yb_h), y_ref, terms, BF16_TOL, what + " bf16")
    assert_bitwise(yb_h, F.f32_to_bf16_bits(yf_h), what + " bf16 = rne(f32)")


def test_w8a16_batch_invariance():
    """A row's bits alone and in batches of 2, 5 and 16 rows."""
    N, K = 96, 2048
    wq, sw, x = _w8_case(31, 16, N, K)
    xb = F.f32_to_bf16_bits(x)
    _, y16 = q4.q8_linear_w8a16(dev(xb), dev(wq), dev(sw), want_f32=True)
    y16 = host(y16)
    for M in (1, 2, 5):
        _, y = q4.q8_linear_w8a16(dev(xb[:M]), dev(wq), dev(sw), want_f32=True)
        assert_bitwise(host(y), y16[:M], f"first {M} rows")


def test_w8_k_zero():
    y = q4.q8_linear_w8a32(dev(np.zeros((3, 1), np.float32))[:, :0].contiguous(), dev(np.zeros((5, 1), np.int8))[:, :0].contiguous(),
                           dev(np.ones(5, np.float32)))
    assert np.array_equal(host(y), np.zeros((3, 5), np.float32))


# --------------------------------------------------------------------------
# the library's own all-extreme route checks ("ftts_kernels" module int8,
# "Tier law")
# --------------------------------------------------------------------------

def test_selftest_all_routes():
    """q4_selftest runs all-extreme rows through every route at the largest
    K each accepts and compares every output with its closed form."""
    report = q4.q4_selftest()
    n = int(report.split()[0])
    assert "passed" in report and n >= 45, report
    # the tiled kernel's per-channel limit and the API's K limit are exercised
    assert "per channel, tiled K=131072" not in report and "per channel, generic" not in report, report


# --------------------------------------------------------------------------
# seeded random shapes across the route thresholds, every route
# --------------------------------------------------------------------------

def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 24, 25, 33, 40, 41, 70]))
        N = int(rng.integers(1, 300))
        G = int(rng.choice([32, 64, 128, 256]))
        K = G * int(rng.integers(1, 24))
        out.append((M, N, K, G))
    return out


@pytest.mark.parametrize("M,N,K,G", _random_shapes(2024, 24))
@_paths("auto", "generic", "gemv", "tiled")
def test_random_shapes_integer_linears(M, N, K, G, path):
    """W4A8 per channel (odd K too), grouped (G = 128 multiples) and W8A8 on
    seeded random shapes: bit-exact against the oracle on every route (a
    forced route that cannot take a shape falls back to the general kernel)."""
    q4.q4_set_path(path)
    c = WL.small_int_case(M * 7919 + N * 31 + K, M, N, K, 0)
    y = q4.q4_linear_w4a8(dev(c["xq"]), dev(c["sx"]), dev(c["w"]), dev(c["sw"]), 0, "excess8")
    assert_bitwise(host(y), L.linear_w4a8(c["xq"], c["sx"], c["w"], c["sw"], 0, F.EXCESS8),
                   f"per channel M{M} N{N} K{K} via {q4.q4_last_path()}")
    Ko = K - 1   # odd K: the pad nibble
    co = WL.small_int_case(M * 7919 + N * 31 + Ko, M, N, Ko, 0)
    y = q4.q4_linear_w4a8(dev(co["xq"]), dev(co["sx"]), dev(co["w"]), dev(co["sw"]), 0, "excess8")
    assert_bitwise(host(y), L.linear_w4a8(co["xq"], co["sx"], co["w"], co["sw"], 0, F.EXCESS8),
                   f"per channel M{M} N{N} K{Ko} via {q4.q4_last_path()}")
    if K % 128 == 0:
        cg = WL.small_int_case(M * 7919 + N * 31 + K + 1, M, N, K, 128)
        y = q4.q4_linear_w4a8(dev(cg["xq"]), dev(cg["sx"]), dev(cg["w"]), dev(cg["sw"]), 128, "twos")
        assert_bitwise(host(y), L.linear_w4a8(cg["xq"], cg["sx"], cg["w"], cg["sw"], 128, F.TWOS),
                       f"grouped M{M} N{N} K{K} via {q4.q4_last_path()}")
    c8 = WL.small_int_case(M * 7919 + N * 31 + K + 2, M, N, K, 0, w_int8=True)
    y = q4.q8_linear_w8a8(dev(c8["xq"]), dev(c8["sx"]), dev(c8["w"]), dev(c8["sw"]))
    assert_bitwise(host(y), L.linear_w8a8(c8["xq"], c8["sx"], c8["w"], c8["sw"]),
                   f"w8a8 M{M} N{N} K{K} via {q4.q4_last_path()}")


@pytest.mark.parametrize("M,N,K,G", _random_shapes(4048, 24))
@_paths("auto", "generic", "gemv", "gemv_mc", "tiled")
def test_random_shapes_float_linears(M, N, K, G, path):
    """W4A16 and W4A32 on seeded random shapes, within tolerance of the
    exact value on every route."""
    q4.q4_set_path(path)
    c = WL.small_float_case(M * 104729 + N * 17 + K + G, M, N, K, G, "excess8")
    yb, yf = q4.q4_linear_w4a16(dev(c["x_bf16"]), dev(c["qweight"]), dev(c["scales_bf16"]), G, "excess8",
                                want_f32=True)
    _w4a16_check(c, yb, yf, f"W4A16 M{M} N{N} K{K} G{G} via {q4.q4_last_path()}")
    ct = WL.small_float_case(M * 104729 + N * 17 + K + G + 1, M, N, K, G, "twos")
    y = q4.q4_linear_w4a32(dev(ct["x_f32"]), dev(ct["qweight"]), dev(ct["scales_f16"], torch.float16), G, "twos")
    y_ref = L.linear_w4a32(ct["x_f32"], ct["qweight"], ct["scales_f16"], G, "twos")
    terms = L.abs_terms(ct["x_f32"].astype(np.float64), ct["qweight"], F.f16_bits_to_float(ct["scales_f16"]), K, G,
                        "twos")
    assert_close(host(y), y_ref, terms, F32_TOL, f"W4A32 M{M} N{N} K{K} G{G} via {q4.q4_last_path()}")


@pytest.mark.parametrize("M,N,K,G", _random_shapes(8096, 16))
@_paths("auto", "generic", "gemv", "tiled")
def test_random_shapes_zero_points(M, N, K, G, path):
    """The zero-point entry points on seeded random shapes and every route:
    W4A8 bit-exact, W4A16 within tolerance (same checks as the fixed cases)."""
    test_w4a8_zero_points_bitwise(M, N, K, G, path)
    test_w4a16_zero_points_tolerance(M, N, K, G, path)


@pytest.mark.parametrize("seed", range(8))
def test_random_multi_problem_lists(seed):
    """q4_linear_w4a8_dynamic_multi on seeded random problem lists: random
    M (1..16), activation type, problem count (1..20), N (0..3000) and K
    (ceil(K/2) a multiple of 16, odd K included, within the LDS limit)."""
    rng = np.random.default_rng(5000 + seed)
    M = int(rng.choice([1, 1, 2, 3, 4, 7, 8, 16]))
    dt = "bf16" if rng.random() < 0.5 else "f32"
    mp = 1 << (M - 1).bit_length()
    shapes = []
    for _ in range(int(rng.integers(1, 21))):
        passes = int(rng.integers(1, max(2, 31 // mp + 1)))
        K = 32 * int(rng.integers(1, 64 * passes + 1)) - int(rng.integers(0, 2))
        while mp * -(-K // 2048) > 31:
            K -= 2048
        shapes.append((int(rng.integers(0, 3001)), max(K, 31)))
    cases = _multi_case(M, dt, shapes, 7000 + seed)
    ys = q4.q4_linear_w4a8_dynamic_multi([(dev(x), dev(w), dev(sw)) for x, w, sw in cases])
    for i, ((x, w, sw), y) in enumerate(zip(cases, ys)):
        y_ref, _, _ = L.linear_w4a8_dynamic(x, w, sw, 0, F.EXCESS8, dt)
        assert_bitwise(host(y), y_ref, f"seed {seed} M{M} {dt} problem {i} N{w.shape[0]} K{x.shape[1]}")
