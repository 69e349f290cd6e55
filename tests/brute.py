"""Brute-force restatements used to pin the CPU oracle.

Each rule is stated in its defining form rather than the oracle's:
rounding is an argmin over every code (ties to the even code), the mask is
the lexicographically smallest valid pair, sums are exact rationals.  Values
are numpy float32/float64; no code is shared with ``oracle/``.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_argmin(t: np.ndarray) -> np.ndarray:
    """E2M1 codes of exact values t (float64): nearest magnitude among the 8,
    ties to the code with mantissa bit 0, sign bit = signbit(t)."""
    t = np.asarray(t, dtype=np.float64)
    # every magnitude above 6 is nearest to 6; clipping keeps float64
    # distances meaningful for huge inputs
    a = np.minimum(np.abs(t), 16.0)[..., None]
    d = np.abs(a - E2M1_MAGS)                        # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among tied candidates prefer an even code (mantissa bit 0)
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return (pick | (np.signbit(t) * 8)).astype(np.uint8)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code).astype(np.int64)
    return E2M1_MAGS[code & 7] * np.where(code & 8, -1.0, 1.0)


def e4m3_table() -> np.ndarray:
    """Values of the 127 non-negative finite E4M3 codes 0x00..0x7E."""
    vals = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


E4M3_VALUES = e4m3_table()


def e4m3_argmin(v: np.ndarray) -> np.ndarray:
    """Nearest non-negative finite E4M3 code, ties to even mantissa; values
    beyond the largest finite magnitude saturate to 0x7E."""
    # every value above 448 is nearest to 448; clip to keep distances exact
    v = np.minimum(np.asarray(v, dtype=np.float64), 1024.0)[..., None]
    d = np.abs(v - E4M3_VALUES)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(0x7F) % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return pick.astype(np.uint8)


def mask_pair_brute(v) -> tuple:
    """Among the 6 index pairs whose kept magnitudes are all >= every dropped
    magnitude, the lexicographically smallest (i0, i1)."""
    a = [abs(float(x)) for x in v]
    for i0 in range(4):
        for i1 in range(i0 + 1, 4):
            kept = [a[i0], a[i1]]
            dropped = [a[j] for j in range(4) if j not in (i0, i1)]
            if min(kept) >= max(dropped):
                return i0, i1
    raise AssertionError("no valid pair")


def mx_quantize_brute(v: np.ndarray):
    """MXFP4 block (exact float64 values): scale exponent e is the one that
    puts the block maximum into the top E2M1 binade [4, 8) (OCP MX floor
    rule), clamped to the E8M0 range; codes by argmin on v / 2^e."""
    v = np.asarray(v, dtype=np.float64)
    amax = float(np.abs(v).max())
    if amax == 0.0:
        e = -127
    else:
        e = -200
        while amax / 2.0 ** e >= 8.0:      # first e with amax / 2^e < 8
            e += 1
        # amax / 2^(e-1) >= 8, so amax / 2^e lies in [4, 8)
        assert 4.0 <= amax / 2.0 ** e < 8.0
        e = max(-127, min(127, e))
    codes = e2m1_argmin(v / 2.0 ** e)
    return codes, e + 127, e2m1_value(codes) * 2.0 ** e


def fraction_dot(a, b) -> Fraction:
    return sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b)), Fraction(0))


# ---------------------------------------------------------------- fp32 steps
# numpy float32 scalars and arrays round every +, -, *, / and sqrt to nearest
# even (IEEE binary32) and never contract a product into an FMA, so these
# restate the fp32 step sequences of the RMSNorm and of the NVFP4-style block
# quantizer with an arithmetic of their own.

def bf16_rne_bits(v) -> np.ndarray:
    """bf16 bit patterns of finite float32 values: the value rounded to its
    8 leading significant bits (or to a multiple of 2^-133 below 2^-126),
    nearest, ties to even, computed on the exact value in float64."""
    v64 = np.asarray(v, dtype=np.float32).astype(np.float64)
    _, e = np.frexp(np.abs(v64))                 # |v| = f 2^e, f in [0.5, 1)
    q = np.maximum(e - 8, -133)                  # weight of the last kept bit
    r = np.ldexp(np.rint(np.ldexp(np.abs(v64), -q)), q)
    out = np.copysign(r, v64).astype(np.float32)   # exact: at most 8 significant bits
    return (out.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_value(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def pairwise_halves_f32(q: np.ndarray) -> np.float32:
    """fl32 sum as a perfect binary tree over the next power of two of
    leaves (missing leaves +0): the sum of a run is the fl32 sum of the sums
    of its two halves."""
    q = np.asarray(q, dtype=np.float32)
    n = 1
    while n < q.size:
        n *= 2
    leaves = np.zeros(n, np.float32)
    leaves[:q.size] = q

    def rec(lo: int, hi: int) -> np.float32:
        if hi - lo == 1:
            return leaves[lo]
        if hi - lo <= 64:                        # small runs: level by level
            a = leaves[lo:hi].copy()
            while a.size > 1:
                a = (a[: a.size // 2 * 2].reshape(-1, 2)[:, 0]
                     + a[: a.size // 2 * 2].reshape(-1, 2)[:, 1]).astype(np.float32)
            return np.float32(a[0])
        mid = (lo + hi) // 2
        return np.float32(rec(lo, mid) + rec(mid, hi))

    return rec(0, n)


def rms_reciprocal_f32(x_bits, eps: float) -> np.float32:
    """r of the RMSNorm of one bf16 row: 1 / sqrt(sum(x^2) / K + eps), each
    step one binary32 operation, the sum a perfect binary tree."""
    x = bf16_bits_value(x_bits).ravel()
    ss = pairwise_halves_f32((x * x).astype(np.float32))
    mean = np.float32(ss / np.float32(x.size))
    s = np.sqrt(np.float32(mean + np.float32(eps)), dtype=np.float32)
    return np.float32(np.float32(1.0) / s)


def rmsnorm_f32(x_bits, g_bits, r) -> np.ndarray:
    """(x * r) * gamma in binary32, before the rounding to bf16."""
    x = bf16_bits_value(x_bits)
    g = bf16_bits_value(g_bits)
    return ((x * np.float32(r)).astype(np.float32) * g).astype(np.float32)


def nv_block_brute(v, s_t):
    """NVFP4-style block of float32 values under tensor scale s_t: E4M3 scale
    code = nearest to amax / (6 s_t) (one binary32 division by the binary32
    product 6 s_t), S = e4m3 value * s_t (binary32), element codes = nearest
    E2M1 to the binary32 quotient v / S; S == 0 gives signed zeros."""
    v = np.asarray(v, dtype=np.float32)
    s_t = np.float32(s_t)
    amax = np.float32(np.abs(v).max())
    ratio = np.float32(amax / np.float32(np.float32(6.0) * s_t))
    sb = int(e4m3_argmin(np.float64(ratio)))
    S = np.float32(np.float32(E4M3_VALUES[sb]) * s_t)
    if S == 0:
        c = (np.signbit(v) * 8).astype(np.uint8)
        return c, sb, np.where(np.signbit(v), -0.0, 0.0).astype(np.float32)
    t = (v / S).astype(np.float32)
    c = e2m1_argmin(t.astype(np.float64))
    return c, sb, (e2m1_value(c).astype(np.float32) * S).astype(np.float32)
