"""The mutation check's plants exist where tests/kernel_mutants.py says, and
are all behind the compile-time switch (CPU only; the check itself builds
and runs the mutant libraries on the GPU)."""
import os
import re

from tests.kernel_mutants import MUTANTS

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "int4_dequantize_matmul_amd", "csrc")


def test_every_mutant_is_planted_in_its_file():
    for n, (src, _) in MUTANTS.items():
        text = open(os.path.join(CSRC, src)).read()
        assert re.search(rf"Q4_MUTANT [!=]= {n}\b", text), f"mutant s{n:02d} not planted in {src}"


def test_switch_defaults_off():
    hdr = open(os.path.join(CSRC, "q4_device.hpp")).read()
    assert "#ifndef Q4_MUTANT\n#define Q4_MUTANT 0\n#endif" in hdr
    build = open(os.path.join(os.path.dirname(CSRC), "build.py")).read()
    assert "Q4_MUTANT" not in build   # the shipped library is built with no mutant
