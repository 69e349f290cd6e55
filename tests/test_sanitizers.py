"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code (CPU).

* The CPU oracle, built with gcc -fsanitize=address,undefined together with
  tests/host/oracle_sanitize_main.c, which drives every oracle entry point on
  small and edge-case inputs (zeros, subnormal squares, values near the top
  of the range, non-power-of-two K, both formats).
* The C ABI's host code (sharq_abi.cpp: validation, view decoding and
  dispatch), built for the host alone with g++ and the same sanitizers, the
  HIP launches replaced by counting stubs (tests/host/abi_launch_stub.cpp);
  tests/test_abi_host.py runs against it, then valid requests of every kind
  that reach the stubs.
Any sanitizer report aborts the run and fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sparsity_fp4_quantized_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc/g++ not installed")


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "host", "oracle_sanitize_main.c"),
                    os.path.join(ROOT, "oracle", "sharq_oracle.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle sanitize run ok" in r.stdout


def test_abi_host_code_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan) or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("sanitizer runtimes or HIP headers missing")
    lib = str(tmp_path / "libsharq_hostsan.so")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", CSRC, "-o", lib, os.path.join(CSRC, "sharq_abi.cpp"),
                    os.path.join(HERE, "host", "abi_launch_stub.cpp")], check=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "host", "run_abi_sanitized.py"), lib],
                       capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "abi sanitize run ok" in r.stdout
