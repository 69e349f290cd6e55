"""The oracle's fp32 step sequences against restatements in numpy float32.

The RMSNorm the SharQ preparation absorbs (arXiv:2606.26587, abstract,
sentence 5) and the NVFP4-style block quantizer (sentence 7) are sequences of
binary32 operations whose order decides the bits.  tests/brute.py states each
sequence again with numpy's binary32 arithmetic (a recursive-halves tree sum,
IEEE division and square root), and these tests require bit equality with the
oracle: on random rows with non-unit gains, and on blocks searched for inputs
where a plausible reordering of the steps (a product reassociated, a division
replaced by a reciprocal multiply, a sequential sum) changes the result.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from brute import (E4M3_VALUES, bf16_rne_bits, e2m1_argmin, e4m3_argmin, mx_quantize_brute,
                   nv_block_brute, rms_reciprocal_f32, rmsnorm_f32)

f32 = np.float32


def _rows(rng, m, k):
    """bf16 rows with magnitudes spread over many binades, some outliers."""
    base = rng.standard_t(4, (m, k)) * 10.0 ** rng.uniform(-3, 3, (m, 1))
    cols = rng.choice(k, max(1, k // 100), replace=False)
    base[:, cols] *= 50.0
    return si.f32_to_bf16_bits(base.astype(np.float32))


def _gains(rng, k, spread):
    g = 1.0 + spread * rng.standard_normal(k) if spread < 1 else 10.0 ** rng.uniform(-2, 2, k)
    return si.f32_to_bf16_bits(g.astype(np.float32))


# ------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("k", [32, 96, 1000, 4096, 14336])
@pytest.mark.parametrize("eps", [1e-5, 1e-6, 0.375])
def test_rms_reciprocal_bitwise(k, eps):
    rng = np.random.default_rng(k + int(eps * 1e6))
    x = _rows(rng, 24, k)
    for i in range(x.shape[0]):
        got = oracle.rms_reciprocal(x[i], eps)
        want = rms_reciprocal_f32(x[i], eps)
        assert got.view(np.uint32) == want.view(np.uint32), (k, eps, i, got, want)


def test_rms_reciprocal_special_rows():
    k = 96
    zero = np.zeros(k, np.uint16)
    assert oracle.rms_reciprocal(zero, 1e-5) == f32(1) / np.sqrt(f32(1e-5), dtype=np.float32)
    # one huge element: its square dominates; tiny ones underflow to fp32 subnormals
    x = np.zeros(k, np.float32)
    x[3], x[50] = 3e18, 1e-30
    xb = si.f32_to_bf16_bits(x)
    assert oracle.rms_reciprocal(xb, 1e-5) == rms_reciprocal_f32(xb, 1e-5)


@pytest.mark.parametrize("k,spread", [(96, 0.1), (4096, 0.1), (1000, 5.0), (14336, 0.3)])
def test_rmsnorm_scale_and_rounding_bitwise(k, spread):
    rng = np.random.default_rng(7 * k)
    x = _rows(rng, 16, k)
    g = _gains(rng, k, spread)
    xn = oracle.normalize(x, g, 1e-5)
    for i in range(x.shape[0]):
        r = rms_reciprocal_f32(x[i], 1e-5)
        y = rmsnorm_f32(x[i], g, r)
        got = oracle.rmsnorm_scale(x[i], g, r)
        assert np.array_equal(got.view(np.uint32), y.view(np.uint32)), (k, i)
        assert np.array_equal(xn[i], bf16_rne_bits(y)), (k, i)


# ------------------------------------------------------------ NVFP4-style block
MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _near(v: np.ndarray, ulps: int) -> np.ndarray:
    """float32 values within `ulps` units in the last place of v (positive v)."""
    b = v.astype(np.float32).view(np.uint32).astype(np.int64)
    d = np.arange(-ulps, ulps + 1)
    return (b[:, None] + d[None, :]).ravel().astype(np.uint32).view(np.float32)


def _random_st(rng) -> np.float32:
    return f32(rng.uniform(1.0, 2.0) * 2.0 ** int(rng.integers(-24, 24)))


def _quotient_alternatives(v, S, sbv, s_t):
    """Plausible other fp32 orders for t = v / S."""
    one = f32(1)
    return [
        (v * f32(one / S)).astype(np.float32),                       # reciprocal multiply
        ((v / f32(sbv)).astype(np.float32) / s_t).astype(np.float32),   # two divisions
        (v.astype(np.float64) / (float(sbv) * float(s_t))).astype(np.float32),   # one rounding of the exact quotient by e4m3 * s_t
    ]


def division_sensitive_blocks(seed: int, want: int):
    """(block, s_t) pairs where some element's E2M1 code under t = fl32(v / S)
    differs from its code under one of the alternatives: elements within a
    few ulps of midpoint * S; the block's first element fixes the E4M3 scale."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < want:
        s_t = _random_st(rng)
        sb = int(rng.integers(1, 127))
        sbv = f32(E4M3_VALUES[sb])
        S = f32(sbv * s_t)
        d6 = f32(f32(6) * s_t)
        amax = f32(sbv * d6)
        if not np.isfinite(amax) or S == 0 or int(e4m3_argmin(np.float64(f32(amax / d6)))) != sb:
            continue
        v = _near((MIDPOINTS * np.float64(S)).astype(np.float32), 3)
        v = v[(v > 0) & (v <= amax)]
        t = (v / S).astype(np.float32)
        code = e2m1_argmin(t.astype(np.float64))
        hit = np.zeros(v.size, bool)
        for alt in _quotient_alternatives(v, S, sbv, s_t):
            hit |= e2m1_argmin(alt.astype(np.float64)) != code
        v = v[hit]
        if v.size == 0:
            continue
        v = v[:15] * np.where(rng.random(min(15, v.size)) < 0.5, f32(-1), f32(1))
        block = np.concatenate([[amax], v, (rng.uniform(-1, 1, 15 - v.size) * amax).astype(np.float32)])
        out.append((block.astype(np.float32), s_t))
    return out


def _ratio_alternatives(amax, s_t):
    six = f32(6)
    return [
        f32(f32(amax / six) / s_t),
        f32(amax * f32(f32(1) / f32(six * s_t))),
        f32(np.float64(amax) / (6.0 * np.float64(s_t))),
    ]


def ratio_sensitive_blocks(seed: int, want: int):
    """(block, s_t) pairs whose E4M3 scale code under fl32(amax / fl32(6 s_t))
    differs from its code under one of the alternative orders: amax within a
    few ulps of an E4M3 midpoint times 6 s_t."""
    rng = np.random.default_rng(seed)
    mids = (E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2.0
    out = []
    while len(out) < want:
        s_t = _random_st(rng)
        d6 = f32(f32(6) * s_t)
        for a in _near((mids * np.float64(d6)).astype(np.float32), 2):
            if not np.isfinite(a) or a <= 0:
                continue
            sb = int(e4m3_argmin(np.float64(f32(a / d6))))
            if any(int(e4m3_argmin(np.float64(r))) != sb for r in _ratio_alternatives(a, s_t)):
                rest = (rng.uniform(-1, 1, 15) * a).astype(np.float32)
                out.append((np.concatenate([[a], rest]).astype(np.float32), s_t))
    return out[:want]


def _check_nv_blocks(cases):
    for block, s_t in cases:
        c, sb, d = oracle.nv_block(block, s_t)
        wc, wsb, wd = nv_block_brute(block, s_t)
        assert sb == wsb, (block, s_t, sb, wsb)
        assert np.array_equal(c, wc), (block, s_t, c, wc)
        assert np.array_equal(d.view(np.uint32), wd.view(np.uint32)), (block, s_t)


def test_nv_block_division_sensitive():
    cases = division_sensitive_blocks(11, 300)
    assert len(cases) == 300
    _check_nv_blocks(cases)


def test_nv_block_ratio_sensitive():
    cases = ratio_sensitive_blocks(12, 300)
    assert len(cases) == 300
    _check_nv_blocks(cases)


def test_nv_block_ties_random_and_degenerate():
    rng = np.random.default_rng(13)
    cases = []
    # power-of-two tensor scales: S has at most 4 significant bits, so
    # midpoint * S is exact and t lands on the tie itself
    for j in range(-10, 11, 5):
        s_t = f32(2.0 ** j)
        for sb in range(1, 127, 5):
            S = np.float64(E4M3_VALUES[sb]) * 2.0 ** j
            v = np.concatenate([[6 * S], MIDPOINTS * S, -MIDPOINTS * S, [0.0]]).astype(np.float32)
            cases.append((np.resize(v, 16), s_t))
    for _ in range(200):
        s_t = _random_st(rng)
        cases.append(((rng.standard_t(4, 16) * float(s_t) * 10.0 ** rng.uniform(-2, 3)).astype(np.float32), s_t))
    cases.append((np.zeros(16, np.float32), f32(1)))                                     # S == 0
    cases.append((np.array([-0.0] * 8 + [0.0] * 8, np.float32), f32(0.5)))               # signed zeros
    cases.append(((rng.standard_normal(16) * 1e-38).astype(np.float32), f32(1e-40)))     # subnormal S
    cases.append(((rng.uniform(-1, 1, 16) * 3.3e38).astype(np.float32), f32(3.3e38 / 2688)))   # huge S
    cases.append((np.full(16, 500.0, np.float32), f32(0.01)))                            # ratio beyond 448
    _check_nv_blocks(cases)


def test_mx_block_vs_brute():
    rng = np.random.default_rng(14)
    for _ in range(300):
        v = (rng.standard_t(4, 32) * 10.0 ** rng.uniform(-30, 30)).astype(np.float32)
        c, sb, d = oracle.mx_block(v)
        wc, wsb, wd = mx_quantize_brute(v.astype(np.float64))
        assert sb == wsb and np.array_equal(c, wc) and np.array_equal(d, wd.astype(np.float32))
