"""Host logic of the measured route plan (q4_route_plan): the route and the
tiled work split a call shape gets, computed on the host with no device work.

The plan's crossings were measured on MI355X with both routes forced; these
tests check what must hold whatever the measured numbers are: decode rows
first and tiled rows after the crossing, W4A16 batches of at most 16 rows on
the batch-invariant decode kernel, tiles covered exactly once by the work
split, forced routes honoured, and the call's own argument rules.
"""
import pytest

import int4_dequantize_matmul_amd as q4

CUS = 256          # compute units of an MI355X
SLOTS = 2 * CUS    # tiled workgroups resident at once (two per CU)
SHAPES = [(2048, 2048), (5632, 2048), (13312, 2048), (26624, 2048), (2048, 5632), (13312, 5632),
          (96, 1024), (4096, 4096), (65536, 8192), (1000, 256)]


@pytest.fixture(autouse=True)
def _auto():
    q4.q4_set_path("auto")
    yield
    q4.q4_set_path("auto")


def plan(op, M, N, K, G=0):
    return q4.q4_route_plan(op, M, N, K, G, CUS)


def status(op, M, N, K, G=0, cus=CUS):
    try:
        q4.q4_route_plan(op, M, N, K, G, cus)
    except q4.Q4Error as e:
        return e.status
    return q4.OK


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("op,G", [("w4a8", 0), ("w4a8", 128), ("w4a8_zp", 128), ("w4a16", 128),
                                  ("w4a16_zp", 128)])
def test_decode_rows_then_tiled(op, G, N, K):
    dmax = plan(op, 1, N, K, G)["decode_max"]
    assert 16 <= dmax <= 1024
    for M in sorted({1, 2, 8, 16, dmax // 2, dmax}):
        assert plan(op, M, N, K, G)["path"] == "gemv", (op, M, N, K)
    for M in (dmax + 1, dmax + 17, 2 * dmax + 3, 4096):
        p = plan(op, M, N, K, G)
        assert p["path"] == "tiled", (op, M, N, K)
        assert p["decode_max"] == dmax


@pytest.mark.parametrize("N,K", SHAPES)
def test_w4a16_batches_of_16_rows_always_decode(N, K):
    """Every M <= 16 takes the streaming decode kernel on every shape, so a
    decode row's bits never depend on its batch."""
    for op in ("w4a16", "w4a16_zp"):
        for M in range(1, 17):
            assert plan(op, M, N, K, 128)["path"] == "gemv"


@pytest.mark.parametrize("op", ["w4a8", "w4a16"])
def test_crossing_falls_as_n_grows(op):
    """More output columns give the tiled kernel more workgroups and the
    decode kernels more bytes to reread per 16 rows: at a fixed K the
    crossing never rises with N."""
    for K in (2048, 5632):
        ds = [plan(op, 1, N, K, 128)["decode_max"] for N in (1024, 2048, 5632, 13312, 26624, 65536)]
        assert ds == sorted(ds, reverse=True), (K, ds)


@pytest.mark.parametrize("op", ["w4a8", "w4a16", "w4a16_zp"])
@pytest.mark.parametrize("M", [17, 20, 32, 33, 40, 64, 65, 100, 128, 129, 300, 2048, 72 * 128 - 5, 89 * 128 - 7])
@pytest.mark.parametrize("N", [96, 1000, 1024, 2048, 5632, 13312, 26624, 65536])
def test_tiled_split_covers_every_tile_once(op, M, N):
    q4.q4_set_path("tiled")
    p = plan(op, M, N, 2048, 128)
    assert p["path"] == "tiled"
    tiles = -(-M // 128) * -(-N // 128)
    if op != "w4a8" and (M <= 64 or tiles * 4 <= SLOTS):
        # W4A16 small calls: 64 x 64 pieces only, four per tile
        assert p["whole_tiles"] == 0 and p["piece_rows"] == 64
        assert p["pieces"] == -(-M // 64) * -(-N // 64)
        return
    if p["pieces"] == 0:
        assert p["whole_tiles"] == tiles and p["piece_rows"] == 0
        return
    per_tile = 128 // p["piece_rows"]
    assert p["piece_rows"] in ((32, 64) if op == "w4a8" else (64,))
    assert p["pieces"] % per_tile == 0
    assert p["whole_tiles"] + p["pieces"] // per_tile == tiles
    if M <= 64 or tiles * 4 <= SLOTS:
        # small calls: every tile in pieces (W4A8: 32 rows while all pieces
        # fit one round)
        assert p["whole_tiles"] == 0
        if op == "w4a8":
            assert p["piece_rows"] == (32 if tiles * 4 <= SLOTS else 64)
    else:
        # only the tiles past the last whole round, when they fill at most
        # half of one, in halves
        rem = tiles % SLOTS
        assert p["whole_tiles"] == tiles - rem and 0 < rem * 2 <= SLOTS
        assert p["piece_rows"] == 64


@pytest.mark.parametrize("op", ["w4a8", "w4a16"])
def test_prefill_split(op):
    """M = 2048, N = 13312: 1664 tiles, three whole rounds of 512, and the
    last 128 tiles in 256 half tiles."""
    p = plan(op, 2048, 13312, 2048, 128)
    assert p == {"path": "tiled", "decode_max": p["decode_max"], "whole_tiles": 1536, "piece_rows": 64,
                 "pieces": 256}


def test_other_ops_always_decode():
    for M in (1, 16, 17, 300):
        assert plan("w4a32", M, 2048, 2048, 128)["path"] == "gemv"
        assert plan("w8a8", M, 2048, 2048)["path"] == "gemv"
    assert plan("w4a32", 1, 2048, 2048, 128)["decode_max"] == 2 ** 31 - 1
    assert plan("w8a8", 1, 2048, 2048)["decode_max"] == 2 ** 31 - 1


def test_per_channel_odd_k_never_tiled():
    for M in (1, 4, 17, 500):
        assert plan("w4a8", M, 3072, 1023, 0)["path"] in ("gemv", "generic")
        assert plan("w4a8", M, 3072, 1023, 0)["path"] != "tiled"


def test_forced_routes():
    q4.q4_set_path("generic")
    assert plan("w4a8", 300, 13312, 2048, 128)["path"] == "generic"
    q4.q4_set_path("gemv")
    assert plan("w4a8", 300, 13312, 2048, 128)["path"] == "gemv"
    q4.q4_set_path("tiled")
    assert plan("w4a8", 1, 13312, 2048, 128)["path"] == "generic"    # tiled starts at 17 rows
    assert plan("w4a8", 17, 13312, 2048, 128)["path"] == "tiled"
    q4.q4_set_path("gemv_mc")
    assert plan("w4a16", 8, 13312, 2048, 128)["path"] == "gemv_mc"
    assert plan("w4a16_zp", 8, 13312, 2048, 128)["path"] == "gemv"   # no zero points on that route


def test_empty_and_k_zero():
    assert plan("w4a8", 0, 13312, 2048, 128)["path"] == "auto"
    assert plan("w4a16", 5, 0, 2048, 128)["path"] == "auto"
    assert plan("w4a8", 5, 16, 0, 0)["path"] == "generic"
    assert plan("w4a16", 5, 16, 0, 128)["path"] == "generic"


def test_plan_argument_rules():
    assert status("w4a8", -1, 16, 128) == q4.EINVAL
    assert status("w4a8", 1, 16, 128, G=-128) == q4.EINVAL
    assert status("w4a8", 1, 16, 128, cus=-1) == q4.EINVAL
    assert q4.raw().q4_route_plan(9, 1, 16, 128, 0, CUS, None) == q4.EINVAL
    assert status("w4a16", 1, 16, 127, G=128) == q4.ESHAPE
    assert status("w4a16", 1, 16, 256, G=0) == q4.ESHAPE
    assert status("w4a8", 1, 16, 384, G=256) == q4.ESHAPE
    assert status("w4a8_zp", 1, 16, 256, G=0) == q4.ESHAPE
    assert status("w4a8", 1, 16, q4.W4A8_MAX_K + 2, G=0) == q4.ESHAPE
    assert status("w8a8", 1, 16, q4.W8A8_MAX_K + 1) == q4.ESHAPE
    assert status("w4a8", 1, 16, 1023, G=0) == q4.OK
