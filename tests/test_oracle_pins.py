"""The oracle against what the pages and mathematics fix (CPU only).

Covers the worked example on every linear, every nibble code, the f16 and
bf16 formats, the quantizer contract (ties to even, no most-negative code,
exact negation, the odd-K pad), closed forms on all-extreme rows, the index
probe, equality with dequantize-then-matmul, and exact-rational brute force
on tiny shapes.
"""
import numpy as np
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_PLAIN, ids=lambda f: f.__name__)
def test_pin(check):
    check()


@pytest.mark.parametrize("check", P.ALL_RNG, ids=lambda f: f.__name__)
@pytest.mark.parametrize("seed", [0, 1])
def test_pin_random(check, seed):
    check(np.random.default_rng(seed))
