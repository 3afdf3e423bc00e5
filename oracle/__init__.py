"""Oracle for the fused packed-int4 quantized linear — TEST INFRASTRUCTURE ONLY.

A plain, slow, CPU-only (Python + numpy) statement of what the library
computes, written from the reference pages and pinned by the tests under
``tests/`` against values the pages print, closed forms, invariants and
exact brute force on tiny inputs.  It shares no code with the HIP library and
never imports it; the library never imports this package.  Only the tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use it.

Modules:
  formats   storage formats: nibble packing, the two nibble encodings,
            f16 / bf16 scale decoding, bf16 round-to-nearest-even
  quantize  the symmetric Q4 / Q8 row quantizers
  linear    the four linears (W4A32, W4A16, W4A8 per-channel and grouped,
            W8A8), the dynamic W4A8 composition, the asymmetric
            (per-group zero point) W4A16 and grouped W4A8, and the int8-weight
            float-activation linears W8A32 / W8A16
  errors    the error measures used to judge the float paths

Each public function is tied to facts outside the oracle by at least one
check in tests/oracle_pins.py (values the pages print, closed forms,
invariants, exact-rational replays), and tests/test_oracle_mutants.py plants
a plausible mistake in each and requires a check to fail.  Helpers used only
inside the pins (dequantize_w4) are the "obvious recipe" those pins compare
against and are checked with exact rationals there.
"""
from . import errors, formats, linear, quantize  # noqa: F401
