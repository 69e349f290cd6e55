"""GEMM parity check shared by the GPU tests.

Two bounds, both required: the normwise target of the SharQ dual GEMM,
max |dY| / max |Y| <= 1e-3, and an element-wise bound that no fp32
summation order can exceed: |dY| <= 4 K 2^-24 sum_k (|ds w| + |dr w|) per
output, where the sum (with the NVFP4 tensor scales) comes from the oracle's
decoded operands.  Y is a sum of 2K exact products; any order of fp32
additions errs by at most (2K - 1) 2^-24 times the sum of their magnitudes,
and the oracle's own rounding adds 2^-24 |Y|, so the factor 4K leaves a
margin of two.  A NaN, a zeroed or a stale output fails it wherever the
products are not all zero.
"""
from __future__ import annotations

import numpy as np

GEMM_TOL = 1e-3
UNIT = 2.0 ** -24

# worst |dY| / bound per test, printed in the terminal summary (conftest.py)
WORST: dict = {}


def normwise(y, ref) -> float:
    den = np.abs(ref).max() if np.size(ref) else 0.0
    return float(np.abs(np.asarray(y, np.float64) - ref).max() / (den if den > 0 else 1.0)) if np.size(ref) else 0.0


def check_gemm(y, ref, yabs, k: int, label: str = "") -> float:
    """Assert both bounds; returns the worst ratio |dY| / element-wise bound."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    yabs = np.asarray(yabs, np.float64)
    assert y.shape == ref.shape == yabs.shape, (label, y.shape, ref.shape, yabs.shape)
    if y.size == 0:
        return 0.0
    assert np.isfinite(y).all(), (label, "non-finite output")
    err = normwise(y, ref)
    assert err <= GEMM_TOL, (label, "normwise", err)
    diff = np.abs(y - ref)
    bound = 4.0 * k * UNIT * yabs
    ok = diff <= bound
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())} outputs beyond 4K 2^-24 sum|a w|; first at {i}: "
                             f"gpu {y[i]!r} oracle {ref[i]!r} bound {bound[i]!r}")
    pos = bound > 0
    ratio = float((diff[pos] / bound[pos]).max()) if pos.any() else 0.0
    key = label.split(" ")[0] if label else "gemm"
    WORST[key] = max(WORST.get(key, 0.0), ratio)
    return ratio


def bf16_value(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_gemm_bf16(y16, ref, yabs, k: int, label: str = ""):
    """bf16 outputs (bit patterns): each must be the bf16 rounding, nearest
    even, of a value within the element-wise fp32 bound of the oracle's Y
    (|dY| <= 4 K 2^-24 sum|a w|).  Rounding is monotone, so that holds exactly
    when the output lies between the roundings of the bound's two ends (each
    end widened by one fp32 ulp for its own rounding to fp32)."""
    import oracle
    y16 = np.asarray(y16)
    ref = np.asarray(ref, np.float64)
    b = 4.0 * k * UNIT * np.asarray(yabs, np.float64)
    assert y16.shape == ref.shape, (label, y16.shape, ref.shape)
    y = bf16_value(y16)
    assert np.isfinite(y).all(), (label, "non-finite output")
    lo = np.nextafter((ref - b).astype(np.float32), np.float32(-np.inf))
    hi = np.nextafter((ref + b).astype(np.float32), np.float32(np.inf))
    lo_b, hi_b = bf16_value(oracle.round_bf16(lo)), bf16_value(oracle.round_bf16(hi))
    ok = (lo_b <= y) & (y <= hi_b)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{label}: {int((~ok).sum())} bf16 outputs outside the rounded bound; first at {i}: "
                             f"gpu {y[i]!r} oracle {ref[i]!r} allowed [{lo_b[i]!r}, {hi_b[i]!r}]")

