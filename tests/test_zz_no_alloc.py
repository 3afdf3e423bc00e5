"""The no-allocation dynamic W4A8 entry point against the one that takes a
caller workspace (GPU).

q4_linear_w4a8_dynamic_noalloc keeps the activation codes and scales in a
scratch array the library holds per device.  Its output must equal
q4_linear_w4a8_dynamic's bit for bit on every route, including on a second
call right after the first with a smaller input (the array keeps the last
call's contents, so a stale code or scale would show there).
"""
import numpy as np
import pytest
import torch

import int4_dequantize_matmul_amd as q4
import oracle.formats as F
import oracle.linear as L
from int4_dequantize_matmul_amd import workloads as WL
from tests.gpu_util import assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _auto_path():
    q4.q4_set_path("auto")
    yield
    q4.q4_set_path("auto")


def _case(seed, M, N, K, G, dt):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if dt == "bf16":
        x = WL.bf16_bits(x)
    w = rng.integers(0, 256, (N, (K + 1) // 2), dtype=np.uint8)
    if K % 2:
        w[:, -1] = (w[:, -1] & 0x0F) | 0x80           # the pad nibble of an odd row
    sw = rng.uniform(0.002, 0.03, (N, K // G) if G else (N,)).astype(np.float32)
    return x, w, sw


def _both(x, w, sw, G):
    xd, wd, sd = dev(x), dev(w), dev(sw)
    y_ws = q4.q4_linear_w4a8_dynamic(xd, wd, sd, G, "excess8")
    path_ws = q4.q4_last_path()
    y_na = torch.full_like(y_ws, float("nan"))
    q4.q4_linear_w4a8_dynamic_noalloc(xd, wd, sd, G, "excess8", y=y_na)
    assert q4.q4_last_path() == path_ws
    return host(y_na), host(y_ws), path_ws


# (first call, second call with a smaller input): M, N, K, G, activation type
PAIRS = [
    ((512, 1024, 2048, 128, "bf16"), (40, 256, 1024, 128, "f32")),      # tiled, then tiled
    ((300, 700, 1024, 0, "f32"), (5, 96, 1023, 0, "bf16")),            # tiled per channel, then MFMA GEMV
    ((16, 333, 4096, 128, "bf16"), (3, 64, 512, 128, "f32")),          # MFMA GEMV grouped, twice
    ((2048, 512, 2048, 128, "bf16"), (1, 200, 2048, 0, "bf16")),       # 4 MiB of codes, then the fused decode
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_call(first, second):
    for i, (M, N, K, G, dt) in enumerate((first, second)):
        x, w, sw = _case(1000 * i + M + N + K, M, N, K, G, dt)
        y_na, y_ws, path = _both(x, w, sw, G)
        assert_bitwise(y_na, y_ws, f"call {i} M{M} N{N} K{K} G{G} {dt} via {path}")


def test_noalloc_matches_oracle():
    M, N, K, G = 64, 300, 1024, 128
    x, w, sw = _case(7, M, N, K, G, "bf16")
    y_na, _, _ = _both(x, w, sw, G)
    y_ref, _, _ = L.linear_w4a8_dynamic(x, w, sw, G, F.EXCESS8, "bf16")
    assert_bitwise(y_na, y_ref, "noalloc vs oracle")


def test_noalloc_largest_and_too_large():
    # the largest M for K = 2048 within the scratch array, then one row more
    K, N = 2048, 128
    M = (q4.NOALLOC_SCRATCH_BYTES - 256) // K
    while q4.q4_w4a8_dynamic_workspace(M, K) > q4.NOALLOC_SCRATCH_BYTES:
        M -= 1
    x, w, sw = _case(11, M, N, K, 128, "bf16")
    y_na, y_ws, path = _both(x, w, sw, 128)
    assert_bitwise(y_na, y_ws, f"largest M {M} via {path}")
    x2, w2, sw2 = _case(12, M + 1, N, K, 128, "bf16")
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_linear_w4a8_dynamic_noalloc(dev(x2), dev(w2), dev(sw2), 128, "excess8")
    assert e.value.status == q4.ESHAPE
