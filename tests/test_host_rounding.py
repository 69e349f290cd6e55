"""The preparation's binary64 -> bf16 rounding, built for the host, against
the CPU reference on every branch.

SiLU(gate) * up in front of the down projection's preparation (the step next
to the SharQ preparation operator, abstract sentence 5) is rounded once from
binary64 to bf16.  The device function is plain bit arithmetic, so a host
build of the same header (tests/host/bf16_of_double_host.cpp) can be compared
with the oracle's rounding here: NaN, overflow to Inf, the largest binade,
ties, normal values and the bf16 subnormal range.
"""
import ctypes
import os
import struct
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "sparsity_fp4_quantized_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def host_round(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    out = str(tmp_path_factory.mktemp("hostround") / "libhostround.so")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-O2", "-std=c++17",
                    "-fPIC", "-shared", "-I", CSRC, "-o", out,
                    os.path.join(HERE, "host", "bf16_of_double_host.cpp")], check=True,
                   capture_output=True)
    lib = ctypes.CDLL(out)
    lib.host_bf16_of_double.argtypes = [ctypes.c_double]
    lib.host_bf16_of_double.restype = ctypes.c_uint32
    return lib.host_bf16_of_double


def _d(bits: int) -> float:
    return struct.unpack("<d", struct.pack("<Q", bits))[0]


def _cases():
    rng = np.random.default_rng(5)
    vals = [0.0, -0.0, float("inf"), -float("inf"), float("nan"), -float("nan"),
            _d(0x7FF0000000000001), _d(0xFFF8000000000123), _d(0x7FFFFFFFFFFFFFFF),
            2.0 ** 128, -(2.0 ** 128), 1e39, -1e39, 4.8e38, 1e300, -1e300]
    top = (2.0 - 2.0 ** -7) * 2.0 ** 127            # largest finite bf16
    mid = top + 2.0 ** 119                           # tie between it and 2^128: rounds to Inf
    for v in (top, mid, np.nextafter(mid, 0), np.nextafter(mid, 1e40), np.nextafter(top, 0),
              2.0 ** 127, np.nextafter(2.0 ** 128, 0)):
        vals += [float(v), -float(v)]
    for e in (-126, -127, -133, -134, -140):          # the normal / subnormal boundary
        for f in (1.0, 1.5, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 - 2.0 ** -30):
            vals += [f * 2.0 ** e, -f * 2.0 ** e]
    for e in range(-140, 128, 7):                    # ties and their neighbours in many binades
        t = (1.0 + 2.0 ** -8) * 2.0 ** e
        vals += [t, np.nextafter(t, 0), np.nextafter(t, 1e300), -t]
    vals += list(rng.standard_normal(20000) * 10.0 ** rng.uniform(-45, 45, 20000))
    vals += list(rng.standard_normal(5000) * 2.0 ** rng.uniform(120, 132, 5000))
    return vals


def test_bf16_of_double_host_build_matches_oracle(host_round):
    bad = []
    for v in _cases():
        got, want = host_round(float(v)), oracle.f64_to_bf16(float(v))
        if got != want:
            bad.append((v, hex(got), hex(want)))
    assert not bad, bad[:10]


def test_oracle_f64_to_bf16_non_finite_and_overflow():
    assert oracle.f64_to_bf16(float("inf")) == 0x7F80
    assert oracle.f64_to_bf16(-float("inf")) == 0xFF80
    assert oracle.f64_to_bf16(float("nan")) == 0x7FC0
    assert oracle.f64_to_bf16(_d(0xFFFFFFFFFFFFFFFF)) == 0xFFC0      # a payload NaN stays a NaN
    assert oracle.f64_to_bf16(2.0 ** 128) == 0x7F80
    assert oracle.f64_to_bf16(-1e39) == 0xFF80
    top = (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert oracle.f64_to_bf16(top) == 0x7F7F
    assert oracle.f64_to_bf16(top + 2.0 ** 119) == 0x7F80            # the tie rounds to even: Inf
    assert oracle.f64_to_bf16(np.nextafter(top + 2.0 ** 119, 0)) == 0x7F7F
    # silu(g) * u past the fp32 range from finite fp32 gate and up
    x = oracle.silu_mul(np.array([[20.0, -20.0, 3e38]], np.float32), np.array([[3e38, 3e38, 3e38]], np.float32))
    assert x[0][0] == 0x7F80 and x[0][2] == 0x7F80
    assert x[0][1] & 0x8000 and (x[0][1] & 0x7F80) != 0x7F80        # -20 sigmoid(-20) 3e38 is finite


@pytest.fixture(scope="module")
def host_row_mean(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    out = str(tmp_path_factory.mktemp("rowmean") / "librowmean.so")
    subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-O2", "-std=c++17",
                    "-ffp-contract=off", "-fPIC", "-shared", "-I", CSRC, "-o", out,
                    os.path.join(HERE, "host", "row_mean_host.cpp")], check=True, capture_output=True)
    lib = ctypes.CDLL(out)
    lib.host_row_mean_mismatches.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                             ctypes.POINTER(ctypes.c_int64)]
    lib.host_row_mean_mismatches.restype = ctypes.c_int64
    return lib.host_row_mean_mismatches


def test_row_mean_is_the_ieee_quotient(host_row_mean):
    """The normalized preparation's row mean fl32(ss / k) (the RMSNorm step of
    the preparation operator, abstract sentence 5) takes Markstein's
    correction from fl32(1 / k) inside [2^-100, 2^100] and IEEE division
    outside: identical to ss / k for every k = 32 .. 16384 the kernels take,
    over 2^-110 .. 2^110 and the special values."""
    cases = ctypes.c_int64(0)
    bad = host_row_mean(16384, 4000, 12345, ctypes.byref(cases))
    assert cases.value > 2_000_000
    assert bad == 0, f"{bad} of {cases.value} row means differ from ss / k"
