"""Seeded synthetic inputs for the five benchmark workloads.

Only random draws live here, in the shapes, sizes and value distributions of
the workloads; none of the method's arithmetic.  Tests, the smoke check and
the bench draw inputs from these functions, then hand the same arrays to the
library and to the oracle.

Draws use numpy's PCG64 seeded through SeedSequence(seed).spawn(n), children
taken in a fixed order.  A bf16 input is an f32 draw with its top 16 bits
kept (the stored bits are the input, so how they were obtained does not
matter); an f16 scale is numpy's float16 conversion of an f32 draw.

Workloads (sizes as named):
  w4a32_gemv    M=1, N=K=2048, G=32; bytes uniform (two's-complement codes),
                f16 scales U[0.001, 0.02], x f32 N(0,1)
  w4a8_channel  M=4, N=3072, K=1023; W f32 N(0, 0.02) for the row quantizer,
                x f32 N(0,1) for the activation quantizer
  w4a16_gemv    M in {1,4,8}, N=13312, K=2048, G=128; bytes uniform
                (excess-8 codes), bf16 scales U[0.002, 0.03], x bf16 N(0,1)
  w4a8_prefill  M=2048, N=13312, K=2048, G=128; bytes uniform, f32 scales
                holding bf16 values U[0.002, 0.03], x bf16 N(0,1)
  microdecoder  5 layers x {q,k,v,o 2048x2048; gate, up 5632x2048;
                down 2048x5632}, W f32 N(0, 0.02), each x bf16 [1, K] N(0,1)
"""
from __future__ import annotations

import numpy as np

HIDDEN = 2048
INTER = 5632
LAYERS = 5
PASSES = 15
# (name, N, K) of one microdecoder layer, in execution order
LAYER_LINEARS = (("q", HIDDEN, HIDDEN), ("k", HIDDEN, HIDDEN), ("v", HIDDEN, HIDDEN),
                 ("o", HIDDEN, HIDDEN), ("gate", INTER, HIDDEN), ("up", INTER, HIDDEN),
                 ("down", HIDDEN, INTER))


def _gens(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Keep the top 16 bits of each f32 draw (the stored bf16 pattern)."""
    return (np.ascontiguousarray(f32, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_valued_f32(f32: np.ndarray) -> np.ndarray:
    """f32 draws with the low 16 bits cleared (bf16-representable values)."""
    return (np.ascontiguousarray(f32, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def w4a32_gemv(seed=1001, M=1, N=2048, K=2048, G=32):
    gw, gs, gx = _gens(seed, 3)
    return dict(
        qweight=gw.integers(0, 256, (N, K // 2), dtype=np.uint8),
        scales_f16=gs.uniform(0.001, 0.02, (N, K // G)).astype(np.float32).astype(np.float16).view(np.uint16),
        x=gx.standard_normal((M, K), dtype=np.float32),
        G=G, enc="twos", M=M, N=N, K=K)


def w4a8_channel(seed=1002, M=4, N=3072, K=1023):
    gw, gx = _gens(seed, 2)
    return dict(
        W=(gw.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32),
        x=gx.standard_normal((M, K), dtype=np.float32),
        M=M, N=N, K=K)


def w4a16_gemv(seed=1003, Ms=(1, 4, 8), N=13312, K=2048, G=128):
    gens = _gens(seed, 2 + len(Ms))
    gw, gs = gens[0], gens[1]
    xs = {M: bf16_bits(g.standard_normal((M, K), dtype=np.float32)) for M, g in zip(Ms, gens[2:])}
    return dict(
        qweight=gw.integers(0, 256, (N, K // 2), dtype=np.uint8),
        scales_bf16=bf16_bits(gs.uniform(0.002, 0.03, (N, K // G)).astype(np.float32)),
        x=xs, G=G, enc="excess8", N=N, K=K)


def w4a8_prefill(seed=1004, M=2048, N=13312, K=2048, G=128):
    gw, gs, gx = _gens(seed, 3)
    return dict(
        qweight=gw.integers(0, 256, (N, K // 2), dtype=np.uint8),
        scales=bf16_valued_f32(gs.uniform(0.002, 0.03, (N, K // G)).astype(np.float32)),
        x=bf16_bits(gx.standard_normal((M, K), dtype=np.float32)),
        G=G, enc="excess8", M=M, N=N, K=K)


def microdecoder_linears(layers=LAYERS, hidden=HIDDEN, inter=INTER):
    """(layer, name, N, K) for every linear of one pass, in execution order."""
    dims = {"q": (hidden, hidden), "k": (hidden, hidden), "v": (hidden, hidden), "o": (hidden, hidden),
            "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)}
    return [(l, name, *dims[name]) for l in range(layers) for name, _, _ in LAYER_LINEARS]


def microdecoder_linear(index: int, seed=1005, layers=LAYERS, hidden=HIDDEN, inter=INTER):
    """Inputs of linear `index` of one pass: W f32 [N, K] and x bf16 [1, K]."""
    l, name, N, K = microdecoder_linears(layers, hidden, inter)[index]
    gens = _gens(seed, 2 * len(microdecoder_linears(layers, hidden, inter)))
    gw, gx = gens[2 * index], gens[2 * index + 1]
    return dict(layer=l, name=name, N=N, K=K,
                W=(gw.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32),
                x=bf16_bits(gx.standard_normal((1, K), dtype=np.float32)))


def small_float_case(seed, M, N, K, G, enc="excess8", x_bf16=True, scale_range=(0.002, 0.03)):
    """A scaled-down float-activation case with the same structure."""
    gw, gs, gx = _gens(seed, 3)
    s = gs.uniform(scale_range[0], scale_range[1], (N, K // G)).astype(np.float32)
    x = gx.standard_normal((M, K), dtype=np.float32)
    return dict(
        qweight=gw.integers(0, 256, (N, K // 2), dtype=np.uint8),
        scales_bf16=bf16_bits(s), scales_f16=s.astype(np.float16).view(np.uint16),
        x_bf16=bf16_bits(x), x_f32=x, G=G, enc=enc, M=M, N=N, K=K)


def small_int_case(seed, M, N, K, G=0, w_int8=False):
    """A scaled-down integer-activation case: int8 codes and f32 scales."""
    gw, gs, gx, gsx = _gens(seed, 4)
    Kb = K if w_int8 else (K + 1) // 2
    Gn = K // G if G else 1
    return dict(
        w=(gw.integers(-127, 128, (N, K)).astype(np.int8) if w_int8
           else gw.integers(0, 256, (N, Kb), dtype=np.uint8)),
        sw=gs.uniform(0.002, 0.03, (N, Gn) if G else (N,)).astype(np.float32),
        xq=gx.integers(-127, 128, (M, K)).astype(np.int8),
        sx=gsx.uniform(0.001, 0.05, M).astype(np.float32),
        G=G, M=M, N=N, K=K)
