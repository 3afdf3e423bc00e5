"""The activation quotient of the fused W4A8 decode quantizer equals IEEE
division (host check of the device formula; see fast_quotient_check.c)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_quotient_matches_division(tmp_path):
    exe = tmp_path / "fast_quotient_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "fast_quotient_check.c"), "-lm"], check=True)
    r = subprocess.run([str(exe), "3000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatched 0" in r.stdout
