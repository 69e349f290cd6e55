"""Runs the C ABI's host-only tests against a host build of sharq_abi.cpp
made with AddressSanitizer and UndefinedBehaviorSanitizer (launches stubbed,
tests/host/abi_launch_stub.cpp), then a few valid requests that reach the
stubs.  Started by tests/test_sanitizers.py in a process with the sanitizer
runtimes preloaded: python3 run_abi_sanitized.py LIB."""
import ctypes
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import sparsity_fp4_quantized_amd as sq  # noqa: E402


def _buf(nbytes):
    a = np.zeros(nbytes + 256, np.uint8)
    off = (-a.ctypes.data) % 256
    return a, a.ctypes.data + off


def valid_calls(L):
    keep = []

    def mem(n):
        a, p = _buf(n)
        keep.append(a)
        return p

    m, n, k = 64, 256, 256
    V = sq.FP4ViewC

    def view(rows, kk, sparse, fmt=sq.MXFP4, ts=None, dense=False):
        v = V()
        blk = sq.BLOCK[fmt]
        v.codes, v.ld_codes = mem(rows * kk // (4 if sparse else 2)), kk // (4 if sparse else 2)
        v.meta, v.ld_meta = (mem(rows * kk // 8), kk // 8) if sparse else (None, 0)
        v.scales, v.ld_scales = mem(rows * kk // blk), kk // blk
        v.layout, v.reserved = sq.LAYOUT_ROW_MAJOR, 0
        v.dense_codes, v.ld_dense = (mem(rows * kk // 2), kk // 2) if dense else (None, 0)
        v.tensor_scale = ts
        return v

    before = L.sharq_stub_launches()
    for fmt in (sq.MXFP4, sq.NVFP4):
        ts = mem(8) if fmt == sq.NVFP4 else None
        sp, rs = view(m, k, True, fmt, ts, dense=True), view(m, k, False, fmt, ts)
        w = view(n, k, False, fmt, mem(8) if fmt == sq.NVFP4 else None)
        x, g, y = mem(m * k * 2), mem(k * 2), mem(m * n * 4)
        assert L.sharq_prepare(fmt, x, m, k, k, g, ctypes.c_float(1e-5), ctypes.byref(sp), ctypes.byref(rs), None) == 0
        assert L.sharq_prepare(fmt, x, m, k, k, None, ctypes.c_float(1e-5), ctypes.byref(sp), ctypes.byref(rs), None) == 0
        assert L.sharq_prepare_noalloc(fmt, x, m, k, k, g, ctypes.c_float(1e-5), ctypes.byref(sp), ctypes.byref(rs),
                                       None) == 0
        assert L.sharq_quantize_weight(fmt, mem(n * k * 2), n, k, k, ctypes.byref(w), None) == 0
        variants = (0, 1, 2, 3)
        for v in variants:
            assert L.sharq_dual_gemm(fmt, ctypes.byref(sp), ctypes.byref(rs), ctypes.byref(w), ctypes.byref(w),
                                     m, n, k, y, n, v, None) == 0, (fmt, v)
    mx_sp, mx_rs = view(m, k, True), view(m, k, False)
    assert L.sharq_prepare_residual(sq.MXFP4, mem(m * k * 2), k, mem(m * k * 2), k, mem(m * k * 2), k, m, k,
                                    mem(k * 2), ctypes.c_float(1e-5), ctypes.byref(mx_sp), ctypes.byref(mx_rs),
                                    None) == 0
    assert L.sharq_prepare_silu_mul(sq.MXFP4, mem(m * k * 4), k, mem(m * k * 4), k, m, k,
                                    ctypes.byref(mx_sp), ctypes.byref(mx_rs), None) == 0
    after = L.sharq_stub_launches()
    assert after - before >= 17, (before, after)
    assert L.sharq_stub_bad() == 0


def main(lib_path):
    sq.LIB_PATH = lib_path
    sq._lib = None
    L = sq.lib()
    L.sharq_stub_launches.restype = ctypes.c_int
    L.sharq_stub_bad.restype = ctypes.c_int
    rc = pytest.main(["-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_host.py"),
                      "-k", "not yardstick and not strided and not refuses_without_library"])
    if rc != 0:
        return int(rc)
    valid_calls(L)
    print("abi sanitize run ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
