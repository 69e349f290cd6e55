"""SharQ CPU oracle (ctypes wrapper over ``sharq_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg use this package; the product path (the HIP
library and its Python binding) never imports it, and this package imports
nothing from the product.

The C source states each step and the reading of the SharQ abstract
(arXiv:2606.26587, sentences 3-5 and 7) it follows.  Arrays are numpy;
bf16 values travel as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

MXFP4 = 0
NVFP4 = 1
BLOCK = {MXFP4: 32, NVFP4: 16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sharq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_OMP_LIB_PATH = os.path.join(_HERE, "liboracle_omp.so")

# IEEE binary32 semantics: no contraction into FMA, no fast-math, single thread.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter", "-Wno-unknown-pragmas"]
# The same source for the timed CPU baseline: optimized for the host and with
# the row loops on OpenMP threads; the arithmetic is unchanged (no contraction,
# no fast-math, so every value is the one the plain build computes).
OMP_CFLAGS = ["-O3", "-march=native", "-fopenmp", "-std=c11", "-fPIC", "-shared",
              "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_omp(force: bool = True) -> str:
    """Compile the OpenMP build used by the benchmark's CPU baseline into
    ``oracle/liboracle_omp.so``."""
    if force or not os.path.exists(_OMP_LIB_PATH):
        tmp = _OMP_LIB_PATH + ".tmp"
        subprocess.run(["gcc", *OMP_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _OMP_LIB_PATH)
    return _OMP_LIB_PATH


_lib = None


def _declare(L):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    L.oracle_prepare.argtypes = [ctypes.c_int, P, I64, I64, P, ctypes.c_float,
                                 P, P, P, P, P, P, P]
    L.oracle_prepare.restype = ctypes.c_int
    L.oracle_dual_gemm_pairs.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, P, P, I64,
                                         P, P, I64, P, P, P]
    L.oracle_dual_gemm_pairs.restype = ctypes.c_int
    L.oracle_dual_gemm.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, P, P, I64, I64, I64,
                                   P, P, P]
    L.oracle_dual_gemm.restype = ctypes.c_int
    L.oracle_round_bf16.argtypes = [P, I64, P]
    L.oracle_round_bf16.restype = None
    L.oracle_threads.argtypes = [ctypes.c_int]
    L.oracle_threads.restype = ctypes.c_int
    return L


def omp_lib():
    """The OpenMP build (CPU baseline only): the same C entry points."""
    if not os.path.exists(_OMP_LIB_PATH):
        build_omp(force=False)
    return _declare(ctypes.CDLL(_OMP_LIB_PATH))


_omp_fresh = None


def omp_lib_built():
    """The OpenMP build compiled in this process (-march=native is this host's
    instruction set, so a library built on another machine is not reused)."""
    global _omp_fresh
    if _omp_fresh is None:
        import tempfile
        d = tempfile.mkdtemp(prefix="oracle_omp_")
        path = os.path.join(d, "liboracle_omp.so")
        subprocess.run(["gcc", *OMP_CFLAGS, "-o", path, _SRC, "-lm"], check=True)
        _omp_fresh = _declare(ctypes.CDLL(path))
    return _omp_fresh


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = _declare(ctypes.CDLL(_LIB_PATH))
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_e2m1_encode.argtypes = [ctypes.c_double]
        L.oracle_e2m1_encode.restype = ctypes.c_int
        L.oracle_e2m1_decode.argtypes = [ctypes.c_int]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_mx_scale_exp.argtypes = [ctypes.c_double]
        L.oracle_mx_scale_exp.restype = ctypes.c_int
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_encode.restype = ctypes.c_int
        L.oracle_e4m3_decode.argtypes = [ctypes.c_int]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_tree_sum.argtypes = [P, I64]
        L.oracle_tree_sum.restype = ctypes.c_float
        L.oracle_nv_tensor_scale.argtypes = [ctypes.c_float]
        L.oracle_nv_tensor_scale.restype = ctypes.c_float
        L.oracle_rmsnorm_row.argtypes = [P, P, I64, ctypes.c_float, P]
        L.oracle_rmsnorm_row.restype = None
        L.oracle_rms_reciprocal.argtypes = [P, I64, ctypes.c_float]
        L.oracle_rms_reciprocal.restype = ctypes.c_float
        L.oracle_rmsnorm_scale.argtypes = [P, P, I64, ctypes.c_float, P]
        L.oracle_rmsnorm_scale.restype = None
        L.oracle_mx_block.argtypes = [P, ctypes.c_int, P, P, P]
        L.oracle_mx_block.restype = None
        L.oracle_nv_block.argtypes = [P, ctypes.c_int, ctypes.c_float, P, P, P]
        L.oracle_nv_block.restype = None
        L.oracle_residual_add.argtypes = [P, P, I64, P]
        L.oracle_residual_add.restype = None
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_silu_mul.argtypes = [P, I64, P, I64, I64, I64, P]
        L.oracle_silu_mul.restype = None
        L.oracle_mask_group.argtypes = [P, P, P]
        L.oracle_mask_group.restype = None
        L.oracle_normalize.argtypes = [P, I64, I64, P, ctypes.c_float, P]
        L.oracle_normalize.restype = ctypes.c_int
        L.oracle_residual_f32.argtypes = [ctypes.c_int, P, I64, I64, ctypes.c_float, P]
        L.oracle_residual_f32.restype = ctypes.c_int
        L.oracle_quantize_weight.argtypes = [ctypes.c_int, P, I64, I64, P, P, P]
        L.oracle_quantize_weight.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


# ---------------------------------------------------------------- codecs
def e2m1_encode(t: float) -> int:
    return lib().oracle_e2m1_encode(float(t))


def e2m1_decode(code: int) -> float:
    return lib().oracle_e2m1_decode(int(code))


def mx_scale_exp(amax: float) -> int:
    return lib().oracle_mx_scale_exp(float(amax))


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(float(v))


def e4m3_decode(b: int) -> float:
    return lib().oracle_e4m3_decode(int(b))


def bf16_to_f32(h: int) -> float:
    return lib().oracle_bf16_to_f32(int(h))


def f32_to_bf16(f: float) -> int:
    return lib().oracle_f32_to_bf16(float(f))


def tree_sum(q: np.ndarray) -> np.float32:
    q = np.ascontiguousarray(q, dtype=np.float32)
    return np.float32(lib().oracle_tree_sum(_p(q), q.size))


def nv_tensor_scale(amax: float) -> np.float32:
    return np.float32(lib().oracle_nv_tensor_scale(float(amax)))


def mask_group(v) -> tuple:
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.size == 4
    i0 = ctypes.c_int()
    i1 = ctypes.c_int()
    lib().oracle_mask_group(_p(v), ctypes.byref(i0), ctypes.byref(i1))
    return i0.value, i1.value


# ---------------------------------------------------------------- steps
def normalize(x: np.ndarray, gamma: Optional[np.ndarray], eps: float = 1e-5) -> np.ndarray:
    x = _u16(x)
    m, k = x.shape
    out = np.empty_like(x)
    g = None if gamma is None else _u16(gamma)
    lib().oracle_normalize(_p(x), m, k, _p(g), eps, _p(out))
    return out


def rms_reciprocal(x_row: np.ndarray, eps: float = 1e-5) -> np.float32:
    """r = 1 / sqrt(mean(x^2) + eps) of one bf16 row, as the RMSNorm computes it."""
    x = _u16(x_row).ravel()
    return np.float32(lib().oracle_rms_reciprocal(_p(x), x.size, eps))


def rmsnorm_scale(x_row: np.ndarray, gamma: np.ndarray, r: float) -> np.ndarray:
    """The normalized row in fp32, before its rounding to bf16."""
    x = _u16(x_row).ravel()
    g = _u16(gamma).ravel()
    assert g.size == x.size
    y = np.empty(x.size, np.float32)
    lib().oracle_rmsnorm_scale(_p(x), _p(g), x.size, float(r), _p(y))
    return y


def mx_block(v: np.ndarray):
    """One MXFP4 block of fp32 values: (codes, scale byte, fp32 dequantized values)."""
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    codes = np.zeros(v.size, np.uint8)
    sb = np.zeros(1, np.uint8)
    deq = np.zeros(v.size, np.float32)
    lib().oracle_mx_block(_p(v), v.size, _p(codes), _p(sb), _p(deq))
    return codes, int(sb[0]), deq


def nv_block(v: np.ndarray, s_t: float):
    """One NVFP4-style block of fp32 values under tensor scale s_t:
    (codes, E4M3 scale byte, fp32 dequantized values)."""
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    codes = np.zeros(v.size, np.uint8)
    sb = np.zeros(1, np.uint8)
    deq = np.zeros(v.size, np.float32)
    lib().oracle_nv_block(_p(v), v.size, float(s_t), _p(codes), _p(sb), _p(deq))
    return codes, int(sb[0]), deq


def residual_f32(fmt: int, xn: np.ndarray, s_t: float = 1.0) -> np.ndarray:
    xn = _u16(xn)
    m, k = xn.shape
    r = np.empty((m, k), dtype=np.float32)
    rc = lib().oracle_residual_f32(fmt, _p(xn), m, k, float(s_t), _p(r))
    assert rc == 0
    return r


def prepare(fmt: int, x: np.ndarray, gamma: Optional[np.ndarray] = None, eps: float = 1e-5,
            dense_backbone: bool = False, L=None) -> dict:
    """Preparation operator on X [m, k]; returns the exported arrays.  L: the
    library to run (the OpenMP build for the CPU baseline; default the plain one)."""
    x = _u16(x)
    m, k = x.shape
    blk = BLOCK[fmt]
    out = {
        "meta": np.zeros((m, k // 8), np.uint8),
        "s_codes": np.zeros((m, k // 4), np.uint8),
        "s_scales": np.zeros((m, k // blk), np.uint8),
        "r_codes": np.zeros((m, k // 2), np.uint8),
        "r_scales": np.zeros((m, k // blk), np.uint8),
        "tensor_scale": np.ones(1, np.float32),
    }
    if dense_backbone:
        out["s_dense"] = np.zeros((m, k // 2), np.uint8)
    g = None if gamma is None else _u16(gamma)
    rc = (L or lib()).oracle_prepare(fmt, _p(x), m, k, _p(g), eps, _p(out["meta"]), _p(out["s_codes"]),
                              _p(out["s_scales"]), _p(out["r_codes"]), _p(out["r_scales"]),
                              _p(out.get("s_dense")), _p(out["tensor_scale"]))
    if rc != 0:
        raise ValueError("oracle_prepare: bad arguments")
    return out


def residual_add(h: np.ndarray, o: np.ndarray) -> np.ndarray:
    """x = bf16(fl32(h) + fl32(o)), elementwise (bf16 bit patterns)."""
    h, o = _u16(h), _u16(o)
    assert h.shape == o.shape
    x = np.empty_like(h)
    lib().oracle_residual_add(_p(h), _p(o), h.size, _p(x))
    return x


def prepare_residual(fmt: int, h: np.ndarray, o: np.ndarray, gamma: np.ndarray, eps: float = 1e-5,
                     dense_backbone: bool = False):
    """Residual add, then the preparation operator on the sum: returns the new
    residual stream x = bf16(h + o) and prepare(fmt, x, gamma)."""
    x = residual_add(h, o)
    return x, prepare(fmt, x, gamma, eps, dense_backbone)


def f64_to_bf16(v: float) -> int:
    return lib().oracle_f64_to_bf16(float(v))


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """x = bf16(silu(g) * u) from fp32 gate and up [m, k] (one rounding of a
    binary64 evaluation)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert g.shape == u.shape and g.ndim == 2
    m, k = g.shape
    x = np.empty((m, k), np.uint16)
    lib().oracle_silu_mul(_p(g), k, _p(u), k, m, k, _p(x))
    return x


def prepare_silu_mul(fmt: int, g: np.ndarray, u: np.ndarray, dense_backbone: bool = False):
    """SiLU(gate) * up, then the preparation operator without a norm (the
    down projection's input): returns x and prepare(fmt, x)."""
    x = silu_mul(g, u)
    return x, prepare(fmt, x, None, 1e-5, dense_backbone)


def quantize_weight(fmt: int, w: np.ndarray) -> dict:
    w = _u16(w)
    n, k = w.shape
    blk = BLOCK[fmt]
    out = {
        "codes": np.zeros((n, k // 2), np.uint8),
        "scales": np.zeros((n, k // blk), np.uint8),
        "tensor_scale": np.ones(1, np.float32),
    }
    rc = lib().oracle_quantize_weight(fmt, _p(w), n, k, _p(out["codes"]), _p(out["scales"]),
                                      _p(out["tensor_scale"]))
    if rc != 0:
        raise ValueError("oracle_quantize_weight: bad arguments")
    return out


def _dual_gemm(fmt, prep, wq, want_f64, want_abs, L=None):
    m = prep["r_codes"].shape[0]
    k = prep["r_codes"].shape[1] * 2
    n = wq["codes"].shape[0]
    y = np.zeros((m, n), np.float32)
    y64 = np.zeros((m, n), np.float64) if want_f64 else None
    yabs = np.zeros((m, n), np.float64) if want_abs else None
    (L or lib()).oracle_dual_gemm(fmt, _p(prep["s_codes"]), _p(prep["meta"]), _p(prep["s_scales"]),
                                  _p(prep["r_codes"]), _p(prep["r_scales"]), _p(prep["tensor_scale"]),
                                  _p(wq["codes"]), _p(wq["scales"]), _p(wq["tensor_scale"]),
                                  m, n, k, _p(y), _p(y64), _p(yabs))
    return y, y64, yabs


def dual_gemm(fmt: int, prep: dict, wq: dict, want_f64: bool = False, L=None):
    y, y64, _ = _dual_gemm(fmt, prep, wq, want_f64, False, L)
    return (y, y64) if want_f64 else y


def round_bf16(y) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values, each rounded once to nearest
    even (oracle_round_bf16)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint16)
    lib().oracle_round_bf16(_p(y), y.size, _p(out))
    return out


def dual_gemm_bf16(fmt: int, prep: dict, wq: dict) -> np.ndarray:
    """The dual GEMM's bf16 output: the fp32 Y of ``dual_gemm`` rounded once to
    bf16 (bit patterns, uint16 [m, n])."""
    return round_bf16(dual_gemm(fmt, prep, wq))


def dual_gemm_bound(fmt: int, prep: dict, wq: dict):
    """Y and, per output, the sum of the magnitudes of its 2k products
    (sum_k |ds w| + |dr w|, with the tensor scales): (y, y_abs)."""
    y, _, yabs = _dual_gemm(fmt, prep, wq, False, True)
    return y, yabs


def gather_rows(prep: dict, rows) -> dict:
    """The prepared operands of the listed activation rows (numpy gather)."""
    rows = np.asarray(rows, dtype=np.int64)
    out = {key: np.ascontiguousarray(val[rows]) for key, val in prep.items() if key != "tensor_scale"}
    out["tensor_scale"] = prep["tensor_scale"]
    return out


def expert_rows(wq: dict, e: int, n: int) -> dict:
    """Rows e n .. e n + n - 1 of a stacked weight payload (expert e's W)."""
    out = {key: np.ascontiguousarray(val[e * n:(e + 1) * n]) for key, val in wq.items() if key != "tensor_scale"}
    out["tensor_scale"] = wq.get("tensor_scale", np.ones(1, np.float32))
    return out


def grouped_dual_gemm(fmt: int, prep: dict, row_index, offsets, wq: dict, n: int) -> np.ndarray:
    return grouped_dual_gemm_bound(fmt, prep, row_index, offsets, wq, n)[0]


def grouped_dual_gemm_bound(fmt: int, prep: dict, row_index, offsets, wq: dict, n: int):
    """Grouped dual GEMM (a mixture-of-experts layer's expert GEMMs): grouped
    row i of group e (offsets[e] <= i < offsets[e + 1]) is activation row
    row_index[i] (row i itself when row_index is None), multiplied by group e's
    weight, rows e n .. e n + n - 1 of the stacked payload: per group, the
    dual GEMM of the gathered rows.  Returns Y [offsets[-1], n] and the sums
    of the magnitudes of each output's products."""
    offsets = np.asarray(offsets, dtype=np.int64)
    total = int(offsets[-1])
    idx = np.arange(total) if row_index is None else np.asarray(row_index, dtype=np.int64)
    y = np.zeros((total, n), np.float32)
    yabs = np.zeros((total, n), np.float64)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y[lo:hi], yabs[lo:hi] = dual_gemm_bound(fmt, gather_rows(prep, idx[lo:hi]), expert_rows(wq, e, n))
    return y, yabs


def dual_gemm_silu_prepare(fmt: int, prep: dict, wq: dict, dense_backbone: bool = False):
    """The gate+up projection of a gated MLP followed by the down projection's
    preparation: Y = the dual GEMM of the prepared activations with W
    [2 inter, k], whose first inter rows are the gate and last inter rows the
    up projection (abstract, sentences 4-5); x = bf16(silu(gate) * up) with
    gate = Y[:, :inter] and up = Y[:, inter:] as fp32; then the preparation of
    x without a norm (sentences 3 and 5).  Returns x and prepare(fmt, x)."""
    y = dual_gemm(fmt, prep, wq)
    inter = y.shape[1] // 2
    return prepare_silu_mul(fmt, y[:, :inter], y[:, inter:], dense_backbone)


def grouped_dual_gemm_silu_prepare(fmt: int, prep: dict, row_index, offsets, wq: dict, inter: int,
                                   dense_backbone: bool = False):
    """The grouped gate+up GEMMs of a mixture-of-experts layer followed by the
    down projections' preparation: Y = grouped_dual_gemm with 2 inter rows a
    group (inter gate rows, then inter up rows), then SiLU(gate) * up and the
    preparation of x [rows, inter] without a norm.  Returns x and
    prepare(fmt, x)."""
    y = grouped_dual_gemm(fmt, prep, row_index, offsets, wq, 2 * inter)
    return prepare_silu_mul(fmt, y[:, :inter], y[:, inter:], dense_backbone)


def _dual_gemm_pairs(fmt, prep, wq, rows, cols, want_f64, want_abs):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    k = prep["r_codes"].shape[1] * 2
    y = np.zeros(rows.size, np.float32)
    y64 = np.zeros(rows.size, np.float64) if want_f64 else None
    yabs = np.zeros(rows.size, np.float64) if want_abs else None
    lib().oracle_dual_gemm_pairs(fmt, _p(prep["s_codes"]), _p(prep["meta"]), _p(prep["s_scales"]),
                                 _p(prep["r_codes"]), _p(prep["r_scales"]),
                                 _p(prep["tensor_scale"]), _p(wq["codes"]), _p(wq["scales"]),
                                 _p(wq["tensor_scale"]), k, _p(rows), _p(cols), rows.size,
                                 _p(y), _p(y64), _p(yabs))
    return y, y64, yabs


def dual_gemm_pairs(fmt: int, prep: dict, wq: dict, rows, cols, want_f64: bool = False):
    """Y at the listed (row, col) pairs only (sorted by row is fastest)."""
    y, y64, _ = _dual_gemm_pairs(fmt, prep, wq, rows, cols, want_f64, False)
    return (y, y64) if want_f64 else y


def dual_gemm_pairs_bound(fmt: int, prep: dict, wq: dict, rows, cols):
    """Y at the listed pairs and the sums of the magnitudes of their products."""
    y, _, yabs = _dual_gemm_pairs(fmt, prep, wq, rows, cols, False, True)
    return y, yabs
