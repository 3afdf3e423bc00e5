"""Mutation check of the GPU tests: the pitfalls of "Fused int4 and int8
dequantize-matmul in C", section 5, planted in the HIP kernels.

    python tests/kernel_mutants.py build   # on the build machine (hipcc)
    python tests/kernel_mutants.py run     # on a machine with the GPU

`build` compiles, for each mutant n, the kernel file that carries it with
-DQ4_MUTANT=n (every plant is an `if constexpr (Q4_MUTANT == n)` in that
file; with the switch off the code is unchanged) and links it with the
library's other objects into lib/mutants/libq4_sNN.so.  `run` runs the GPU
test suite once per mutant library (the binding loads the library named by
Q4_LIB) and reports the tests that fail; every mutant must fail at least
one.  s10 and s11 (argument checks) are host code, covered by the CPU tests
of the C ABI; s12 (a thread pool) has no counterpart here.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "int4_dequantize_matmul_amd")
sys.path.insert(0, ROOT)

# mutant: (kernel file, the pitfall as the pages name it)
MUTANTS = {
    1: ("gemv_stream.hip", "nibbles read as unsigned 0..15"),
    2: ("gemv_stream.hip", "the high nibble taken as the even column"),
    3: ("gemv_stream.hip", "scales indexed by group only: every row uses row 0's"),
    4: ("gemm_tiled.hip", "a group's partial sum not reset"),
    5: ("gemv_stream_w4a32.hip", "the f16 scale decoded as bfloat16"),
    6: ("gemv_stream.hip", "codes unpacked at the chunk offset instead of the group's"),
    7: ("gemv_mfma.hip", "the int8 activation scale indexed by the wrong row (row 0's)"),
    8: ("gemv_stream_w4a8.hip", "the int8 activation scale forgotten"),
    9: ("gemv_stream.hip", "a summation order of its own for M = 1"),
}
OUT = os.path.join(PKG, "lib", "mutants")


def lib_path(n):
    return os.path.join(OUT, f"libq4_s{n:02d}.so")


def build():
    from int4_dequantize_matmul_amd import build as B
    B.build()   # the unmutated objects
    os.makedirs(OUT, exist_ok=True)
    for n, (src, _) in MUTANTS.items():
        obj = os.path.join(B.BUILD, f"mutant_s{n:02d}.o")
        B._run([B.HIPCC, *B.HIP_FLAGS, f"-DQ4_MUTANT={n}", "-c", os.path.join(B.CSRC, src), "-o", obj])
        others = [os.path.join(B.BUILD, f) for f in sorted(os.listdir(B.BUILD))
                  if f.endswith(".o") and not f.startswith("mutant_") and f != src + ".o"]
        B._run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib_path(n), obj, *others])
        os.remove(obj)
        print(f"s{n:02d} built", flush=True)


def run(timeout=600):
    rows, missed = [], []
    for n, (src, what) in MUTANTS.items():
        env = dict(os.environ, Q4_LIB=lib_path(n))
        print(f"s{n:02d}: running the GPU tests against {os.path.basename(lib_path(n))}", flush=True)
        r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-m", "gpu", "-q", "-p", "no:cacheprovider",
                            "-rf", "--timeout", "300", "--timeout-method", "thread"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
        failed = sorted(set(re.findall(r"^FAILED (\S+?)(?:\[| |$)", r.stdout, re.M)))
        summary = [l for l in r.stdout.splitlines() if re.search(r"\d+ (passed|failed)", l)]
        print(f"s{n:02d} ({src}): {summary[-1] if summary else r.stdout[-300:]}", flush=True)
        for t in failed[:12]:
            print(f"    {t}", flush=True)
        rows.append((n, src, what, summary[-1] if summary else "?", failed))
        if r.returncode == 0:
            missed.append(n)
    print("mutants not caught:", missed or "none", flush=True)
    return 1 if missed else 0


if __name__ == "__main__":
    if sys.argv[1:] == ["build"]:
        build()
    elif sys.argv[1:] == ["run"]:
        sys.exit(run())
    else:
        print(__doc__)
        sys.exit(2)
