"""The host half of libq4 (quantizers, packer, status strings) built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven over
edge shapes and values (CPU only; "Fused int4 and int8 dequantize-matmul in
C", overview: the C path is tested under ASan and UBSan)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _sanitizers_available(tmp_path):
    probe = tmp_path / "probe.cpp"
    probe.write_text("int main() { return 0; }\n")
    r = subprocess.run(["g++", "-fsanitize=address,undefined", str(probe), "-o", str(tmp_path / "probe")],
                       capture_output=True, text=True)
    return r.returncode == 0


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_asan_and_ubsan(tmp_path):
    if not _sanitizers_available(tmp_path):
        pytest.skip("g++ sanitizer runtimes not installed")
    exe = tmp_path / "host_sanitize_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(HERE, "host_sanitize_check.cpp"),
           os.path.join(ROOT, "int4_dequantize_matmul_amd", "csrc", "q4_host.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ)
    # a preloaded library ahead of the ASan runtime is not an error here
    env["ASAN_OPTIONS"] = "detect_leaks=1:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host sanitizer checks ok" in r.stdout
