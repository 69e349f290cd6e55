"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test ties one oracle step to the OCP value rules, to a brute-force
restatement (tests/brute.py), to a closed form, to an invariant the SharQ
abstract implies (arXiv:2606.26587, sentences 3-5), or to a library routine
(torch's bf16 conversion, numpy matmul, exact rationals).
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from brute import (E2M1_MAGS, E4M3_VALUES, e2m1_argmin, e2m1_value, e4m3_argmin,
                   fraction_dot, mask_pair_brute, mx_quantize_brute)

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
FINITE_BF16 = ALL_BF16[(ALL_BF16 & 0x7F80) != 0x7F80]


def f32(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


# ------------------------------------------------------------ E2M1
def test_e2m1_decode_is_ocp_table():
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for c in range(16):
        v = oracle.e2m1_decode(c)
        assert abs(v) == want[c & 7]
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def test_e2m1_encode_all_bf16_vs_argmin():
    t = si.bf16_bits_to_f32(FINITE_BF16).astype(np.float64)
    got = np.array([oracle.e2m1_encode(v) for v in t], dtype=np.uint8)
    want = e2m1_argmin(t)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(t[i], got[i], want[i]) for i in bad[:10]]


def test_e2m1_encode_midpoints_and_neighbours():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        vals += [m, np.nextafter(m, 0), np.nextafter(m, 10)]
        vals += [-m, -np.nextafter(m, 0), -np.nextafter(m, 10)]
    vals += [0.0, -0.0, 6.0, 7.99, 8.0, 1e30, -1e30, 5e-324, -5e-324]
    t = np.array(vals, dtype=np.float64)
    got = np.array([oracle.e2m1_encode(v) for v in t], dtype=np.uint8)
    assert (got == e2m1_argmin(t)).all()
    # ties go to the even code
    assert oracle.e2m1_encode(0.25) == 0 and oracle.e2m1_encode(0.75) == 2
    assert oracle.e2m1_encode(1.25) == 2 and oracle.e2m1_encode(1.75) == 4
    assert oracle.e2m1_encode(2.5) == 4 and oracle.e2m1_encode(3.5) == 6
    assert oracle.e2m1_encode(5.0) == 6
    # signed zero and negative underflow keep the sign bit
    assert oracle.e2m1_encode(-0.0) == 8 and oracle.e2m1_encode(-0.1) == 8
    assert oracle.e2m1_encode(-100.0) == 15


# ------------------------------------------------------------ E8M0 scale
def test_mx_scale_puts_block_max_in_top_binade():
    # every positive finite bf16 amax, and fp32 edge values
    amaxes = list(si.bf16_bits_to_f32(FINITE_BF16[(FINITE_BF16 & 0x8000) == 0]).astype(np.float64))
    amaxes += [f32(1), f32(0x007FFFFF), f32(0x00800000), f32(0x7F7FFFFF), 2.0 ** -125, 2.0 ** -124]
    for a in amaxes:
        e = oracle.mx_scale_exp(a)
        assert -127 <= e <= 127
        if a == 0.0:
            assert e == -127
            continue
        r = a / 2.0 ** e
        if e > -127:
            assert 4.0 <= r < 8.0, (a, e)
        else:
            assert r < 8.0, (a, e)           # clamped: the block max lands below 8


def test_mx_scale_matches_frexp():
    for a in [1.0, 3.99, 4.0, 7.99, 8.0, 6.0, 0.5, 2.0 ** -126, 2.0 ** -130, 2.0 ** 127]:
        _, E = math.frexp(a)
        assert oracle.mx_scale_exp(a) == max(-127, min(127, (E - 1) - 2))


# ------------------------------------------------------------ E4M3
def test_e4m3_decode_known_values():
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_decode(0x3C) == 1.5
    assert oracle.e4m3_decode(0x00) == 0.0
    got = np.array([oracle.e4m3_decode(b) for b in range(0x7F)])
    assert (got == E4M3_VALUES).all()


def test_e4m3_encode_bf16_and_random_vs_argmin():
    pos = si.bf16_bits_to_f32(FINITE_BF16[(FINITE_BF16 & 0x8000) == 0]).astype(np.float64)
    rng = np.random.default_rng(0)
    rnd = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 20000)).astype(np.float32)
    mids = (E4M3_VALUES[1:] + E4M3_VALUES[:-1]) / 2
    v = np.concatenate([pos, rnd.astype(np.float64), mids, np.nextafter(mids, 0),
                        np.nextafter(mids, 1e9), [448.0, 460.0, 464.0, 1e6]])
    got = np.array([oracle.e4m3_encode(x) for x in v], dtype=np.uint8)
    want = e4m3_argmin(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(v[i], got[i], want[i]) for i in bad[:10]]
    assert oracle.e4m3_encode(1e6) == 0x7E        # saturate, never NaN


# ------------------------------------------------------------ bf16
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]
    ties = (rng.integers(0, 1 << 16, 5000, dtype=np.uint32) << 16) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    allb = np.concatenate([bits, ties]).astype(np.uint32)
    f = allb.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(x)) for x in f[:20000]], dtype=np.uint16)
    assert (got == want[:20000]).all()
    # the generator uses the same rounding; pin it too
    assert (si.f32_to_bf16_bits(f) == want).all()


def test_round_bf16_array_matches_torch():
    """oracle.round_bf16 (the dual GEMM's bf16 output) against torch's fp32 ->
    bf16 conversion on every pattern class: random finite fp32, exact ties
    with even and odd kept bits, subnormals, values that round up into the
    next binade, and values past the largest bf16 that round to infinity."""
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, 300000, dtype=np.uint64).astype(np.uint32)
    hi = rng.integers(0, 1 << 16, 20000, dtype=np.uint32) << 16
    special = np.concatenate([hi | 0x8000, hi | 0x7FFF, hi | 0x8001, hi | 0xFFFF,
                              rng.integers(0, 1 << 23, 5000, dtype=np.uint32),
                              np.array([0x7F7F8000, 0x7F7FFFFF, 0x7F7F7FFF, 0xFF7F8000, 0x00000000,
                                        0x80000000, 0x00008000, 0x00018000], np.uint32)])
    allb = np.concatenate([bits, special]).astype(np.uint32)
    allb = allb[(allb & 0x7F800000) != 0x7F800000]
    f = allb.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_bf16(f), want)
    n2 = f.size // 7 * 7       # a 2-D array keeps its shape
    assert np.array_equal(oracle.round_bf16(f[:n2].reshape(-1, 7)), want[:n2].reshape(-1, 7))


def test_dual_gemm_bf16_exact_product():
    """FP4-grid X and W: the dual GEMM is exact in fp32, so its bf16 output is
    the bf16 rounding (torch's) of the exact product X W^T (numpy, fp64)."""
    m, k, n = 24, 256, 40
    xb = si.fp4_grid(m, k, 0, 21)
    wb = si.fp4_grid(n, k, -6, 22)
    xv = xb.astype(np.uint32) << 16
    wv = wb.astype(np.uint32) << 16
    exact = xv.view(np.float32).astype(np.float64) @ wv.view(np.float32).astype(np.float64).T
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    p = oracle.prepare(oracle.MXFP4, xb, None)
    q = oracle.quantize_weight(oracle.MXFP4, wb)
    got = oracle.dual_gemm_bf16(oracle.MXFP4, p, q)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got, want.view(np.uint16))
    # many of these products are not bf16 values: the rounding is exercised
    assert (exact.astype(np.float32).view(np.uint32) & 0xFFFF).any()


# ------------------------------------------------------------ residual add
def _bf16_pairs(rng, n):
    """Random finite bf16 bit patterns with exponents that keep sums finite,
    plus pairs that cancel and pairs whose sum falls on a bf16 tie."""
    e = rng.integers(60, 190, (2, n)).astype(np.uint32)
    sign = rng.integers(0, 2, (2, n)).astype(np.uint32)
    mant = rng.integers(0, 128, (2, n)).astype(np.uint32)
    b = ((sign << 15) | (e << 7) | mant).astype(np.uint16)
    h, o = b[0], b[1]
    o[:100] = h[:100] ^ 0x8000                       # x + (-x)
    # 1 + 2^-8 (exactly between two bf16 values): ties to even either way
    h[100:110], o[100:110] = 0x3F80, 0x3B80
    h[110:120], o[110:120] = 0x3F81, 0x3B80
    return h, o


def _bf16_rne_exact(v: float) -> int:
    """bf16 bits of the binary32 value v, rounded to 8 significant bits with
    ties to even by way of math.frexp (not the oracle's bit trick)."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    m, e = math.frexp(abs(v))                  # |v| = m 2^e, m in [0.5, 1)
    q = round(m * 256)                         # half to even
    r = math.ldexp(q, e - 8)
    return int(np.float32(math.copysign(r, v)).view(np.uint32) >> 16)


def test_residual_add_vs_exact_sum():
    """bf16(fl32(h + o)): the exact sum (binary64, exact for these exponent
    ranges) rounded to binary32 by numpy, then to bf16 by an independent
    half-to-even rounding."""
    rng = np.random.default_rng(11)
    h, o = _bf16_pairs(rng, 20000)
    got = oracle.residual_add(h, o)
    hf, of = si.bf16_bits_to_f32(h).astype(np.float64), si.bf16_bits_to_f32(o).astype(np.float64)
    want = np.array([_bf16_rne_exact(float(np.float32(a + b))) for a, b in zip(hf, of)], np.uint16)
    assert (got == want).all()
    assert (got[:100] == 0).all()                  # x + (-x) = +0
    assert (got[100:110] == 0x3F80).all() and (got[110:120] == 0x3F82).all()


def test_residual_add_vs_torch_bf16_add():
    """torch's CPU bf16 add (fp32 sum, rounded to bf16) on the same pairs."""
    rng = np.random.default_rng(12)
    h, o = _bf16_pairs(rng, 200000)
    th = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16)
    to = torch.from_numpy(o.view(np.int16)).view(torch.bfloat16)
    want = (th + to).view(torch.int16).numpy().view(np.uint16)
    assert (oracle.residual_add(h, o) == want).all()
    assert (oracle.residual_add(o, h) == want).all()     # commutes


def test_prepare_residual_with_zero_update_is_prepare():
    """o = +0: the residual stream passes through (-0 becomes +0) and the
    preparation is the plain one of h."""
    w = si.WORKLOADS["qkv_prefill"]
    h = si.workload_x(w, m=24)
    h[0, :3] = [0x8000, 0x0000, 0x3F80]
    g = si.gamma(w.k, 77)
    x, p = oracle.prepare_residual(oracle.MXFP4, h, np.zeros_like(h), g, dense_backbone=True)
    want_x = h.copy()
    want_x[want_x == 0x8000] = 0
    assert (x == want_x).all()
    q = oracle.prepare(oracle.MXFP4, want_x, g, dense_backbone=True)
    for key in q:
        assert (p[key] == q[key]).all(), key


# ------------------------------------------------------------ SiLU(gate) * up
def _bf16_of_decimal(v) -> int:
    """bf16 bits nearest (ties to even) to the Decimal v, in Decimal arithmetic."""
    import decimal
    if v == 0:
        return 0x8000 if v.is_signed() else 0
    a = abs(v)
    e = a.adjusted() * 10 // 3 - 2                # a first guess of floor(log2 a)
    two = decimal.Decimal(2)
    while two ** (e + 1) <= a:
        e += 1
    while two ** e > a:
        e -= 1
    e = max(e, -126)                              # bf16 subnormals share 2^-133 steps
    q = (a / two ** (e - 7)).quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_EVEN)
    r = float(q * two ** (e - 7))
    bits = int(np.float32(r).view(np.uint32) >> 16)
    return bits | (0x8000 if v < 0 else 0)


def test_silu_mul_vs_decimal():
    """x = bf16(silu(g) * u): against a 60-digit Decimal evaluation rounded to
    bf16 by Decimal arithmetic, on random fp32 gates and ups over a wide range
    (far from bf16 midpoints the two must agree exactly)."""
    import decimal
    decimal.getcontext().prec = 60
    rng = np.random.default_rng(21)
    g = np.concatenate([rng.normal(0, 3, 3000), rng.uniform(-40, 40, 1000), [0.0, -0.0, 1e-30, -88.0]])
    u = np.concatenate([rng.normal(0, 1, 3000) * 10.0 ** rng.integers(-6, 4, 3000),
                        rng.normal(0, 5, 1000), [3.0, 3.0, 2.0, 1.0]])
    g, u = g.astype(np.float32)[None, :], u.astype(np.float32)[None, :]
    got = oracle.silu_mul(g, u)[0]
    one = decimal.Decimal(1)
    for i in range(g.shape[1]):
        gd, ud = decimal.Decimal(float(g[0, i])), decimal.Decimal(float(u[0, i]))
        v = gd / (one + (-gd).exp()) * ud
        assert got[i] == _bf16_of_decimal(v), (i, float(g[0, i]), float(u[0, i]), hex(got[i]))


def test_silu_mul_closed_forms():
    """silu(0) = 0 (the zero takes u's sign), u = 0 gives a zero with silu's
    sign, and for g = 80 the gate's sigmoid is 1 in every format, so x is the
    product g u rounded once."""
    g = np.array([[0.0, 0.0, 2.0, -2.0, 80.0, 80.0, 95.0]], np.float32)
    u = np.array([[3.0, -3.0, 0.0, 0.0, 1.5, -0.3, 1.0 / 3.0]], np.float32)
    x = oracle.silu_mul(g, u)[0]
    assert list(x[:4]) == [0x0000, 0x8000, 0x0000, 0x8000]
    for i in range(4, 7):
        want = _bf16_of_decimal(__import__("decimal").Decimal(float(g[0, i])) *
                                __import__("decimal").Decimal(float(u[0, i])))
        assert x[i] == want


def test_f64_to_bf16_ties_and_binades():
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80            # tie, even below
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie, even above
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81   # just past the tie
    assert oracle.f64_to_bf16(2.0 - 2.0 ** -9) == 0x4000            # rounds up into the next binade
    assert oracle.f64_to_bf16(-0.0) == 0x8000
    assert oracle.f64_to_bf16(2.0 ** -130) == 0x0008                # bf16 subnormal


# ------------------------------------------------------------ tree sum
def _tree_recursive(q):
    n = len(q)
    if n == 1:
        return np.float32(q[0])
    h = n // 2
    return np.float32(_tree_recursive(q[:h]) + _tree_recursive(q[h:]))


def test_tree_sum_order_example():
    # sequential fp32 summation gives 2^24; the pairwise tree gives 2^24 + 2:
    # (2^24 + 1) rounds to 2^24 (tie to even), (1 + 1) = 2, 2^24 + 2 is exact.
    q = np.array([2.0 ** 24, 1, 1, 1], dtype=np.float32)
    assert float(oracle.tree_sum(q)) == 2.0 ** 24 + 2


def test_tree_sum_integers_exact_and_padding():
    rng = np.random.default_rng(2)
    for n in [1, 3, 7, 32, 100, 256, 1000, 4096, 14336]:
        q = rng.integers(0, 1000, n).astype(np.float32)
        assert float(oracle.tree_sum(q)) == float(q.astype(np.int64).sum())


def test_tree_sum_vs_recursive_halves():
    rng = np.random.default_rng(3)
    for n in [5, 64, 96, 448, 1024]:
        q = (rng.standard_normal(n) ** 2 * rng.choice([1, 1e4, 1e-4], n)).astype(np.float32)
        np2 = 1 << (n - 1).bit_length()
        padded = np.concatenate([q, np.zeros(np2 - n, np.float32)])
        assert oracle.tree_sum(q) == _tree_recursive(padded)


# ------------------------------------------------------------ RMSNorm
def _bf16_ulp(v):
    v = abs(v)
    if v == 0:
        return 2.0 ** -133
    return 2.0 ** (math.floor(math.log2(v)) - 7)


@pytest.mark.parametrize("k", [32, 256, 4096, 96])
def test_rmsnorm_within_one_bf16_ulp_of_fp64(k):
    rng = np.random.default_rng(k)
    x = si.f32_to_bf16_bits((rng.standard_t(4, (4, k)) * 3).astype(np.float32))
    g = si.gamma(k, seed=7)
    xn = oracle.normalize(x, g, 1e-5)
    xf = si.bf16_bits_to_f32(x).astype(np.float64)
    gf = si.bf16_bits_to_f32(g).astype(np.float64)
    ref = xf / np.sqrt((xf ** 2).mean(axis=1, keepdims=True) + 1e-5) * gf
    got = si.bf16_bits_to_f32(xn).astype(np.float64)
    for a, b in zip(got.ravel(), ref.ravel()):
        assert abs(a - b) <= _bf16_ulp(b) * 1.0001, (a, b)


def test_rmsnorm_closed_forms():
    k = 256
    # constant row c: r = 1/sqrt(c^2 + eps); one nonzero entry a: r = 1/sqrt(a^2/k + eps)
    c = 0.75
    x = si.f32_to_bf16_bits(np.full((1, k), c, np.float32))
    g = si.gamma(k, None)
    got = si.bf16_bits_to_f32(oracle.normalize(x, g, 1e-5))[0]
    want = c / math.sqrt(c * c + 1e-5)
    assert np.all(np.abs(got - want) <= _bf16_ulp(want))
    x = np.zeros((1, k), np.float32)
    x[0, 5] = 2.0
    got = si.bf16_bits_to_f32(oracle.normalize(si.f32_to_bf16_bits(x), g, 1e-5))[0]
    want = 2.0 / math.sqrt(4.0 / k + 1e-5)
    assert abs(got[5] - want) <= _bf16_ulp(want)
    assert np.all(got[np.arange(k) != 5] == 0)
    # no gamma: identity
    xb = si.activations("normal", 3, 64, 0, 1.0, 9)
    assert (oracle.normalize(xb, None) == xb).all()


# ------------------------------------------------------------ mask
def test_mask_all_625_groups_vs_brute():
    alphabet = [0.0, 1.0, -1.0, 2.0, -2.0]
    seen = set()
    for a in alphabet:
        for b in alphabet:
            for c in alphabet:
                for d in alphabet:
                    v = [a, b, c, d]
                    got = oracle.mask_group(v)
                    assert got == mask_pair_brute(v), v
                    seen.add(got)
    assert len(seen) == 6


def test_mask_random_groups_and_signed_zero():
    rng = np.random.default_rng(4)
    for _ in range(3000):
        v = rng.standard_normal(4).astype(np.float32)
        v[rng.random(4) < 0.2] = v[0]
        assert oracle.mask_group(v) == mask_pair_brute(v)
    assert oracle.mask_group([-0.0, 0.0, 0.0, -0.0]) == (0, 1)
    assert oracle.mask_group([0.0, 0.0, -0.0, 1.0]) == (0, 3)


# ------------------------------------------------------------ preparation
def _unpack_meta(meta, k):
    m = meta.shape[0]
    nib = np.zeros((m, k // 4), np.uint8)
    nib[:, 0::2] = meta & 15
    nib[:, 1::2] = meta >> 4
    return nib


def _unpack_dense(codes):
    m, kh = codes.shape
    out = np.zeros((m, kh * 2), np.uint8)
    out[:, 0::2] = codes & 15
    out[:, 1::2] = codes >> 4
    return out


def _brute_prepare_mx(xn_bits):
    """Everything after the norm, restated with the brute-force rules."""
    xn = si.bf16_bits_to_f32(xn_bits)
    m, k = xn.shape
    meta = np.zeros((m, k // 4), np.uint8)
    s_dense = np.zeros((m, k), np.uint8)
    s_scale = np.zeros((m, k // 32), np.uint8)
    r_codes = np.zeros((m, k), np.uint8)
    r_scale = np.zeros((m, k // 32), np.uint8)
    for i in range(m):
        v = np.zeros(k, np.float32)
        for g in range(k // 4):
            i0, i1 = mask_pair_brute(xn[i, 4 * g:4 * g + 4])
            meta[i, g] = i0 | (i1 << 2)
            v[4 * g + i0] = xn[i, 4 * g + i0]
            v[4 * g + i1] = xn[i, 4 * g + i1]
        d = np.zeros(k, np.float32)
        for b in range(k // 32):
            c, sb, dq = mx_quantize_brute(v[32 * b:32 * b + 32].astype(np.float64))
            s_dense[i, 32 * b:32 * b + 32] = c
            s_scale[i, b] = sb
            d[32 * b:32 * b + 32] = dq.astype(np.float32)
        r = (xn[i] - d).astype(np.float32)                   # fp32 subtraction
        for b in range(k // 32):
            c, sb, _ = mx_quantize_brute(r[32 * b:32 * b + 32].astype(np.float64))
            r_codes[i, 32 * b:32 * b + 32] = c
            r_scale[i, b] = sb
    return meta, s_dense, s_scale, r_codes, r_scale


@pytest.mark.parametrize("name,rows", [("tiny", 16), ("qkv_prefill", 3), ("down_prefill", 2)])
def test_prepare_mx_vs_brute(name, rows):
    w = si.WORKLOADS[name]
    x = si.workload_x(w, m=rows)
    g = si.workload_gamma(w)
    p = oracle.prepare(oracle.MXFP4, x, g, dense_backbone=True)
    xn = oracle.normalize(x, g)
    meta, s_dense, s_scale, r_codes, r_scale = _brute_prepare_mx(xn)
    k = w.k
    assert (_unpack_meta(p["meta"], k) == meta).all()
    assert (_unpack_dense(p["s_dense"]) == s_dense).all()
    assert (p["s_scales"] == s_scale).all()
    assert (_unpack_dense(p["r_codes"]) == r_codes).all()
    assert (p["r_scales"] == r_scale).all()
    # compressed backbone: code at i0 in the low nibble, code at i1 in the high
    nib = _unpack_meta(p["meta"], k)
    i0, i1 = nib & 3, nib >> 2
    gidx = np.arange(k // 4) * 4
    lo = np.take_along_axis(s_dense, gidx + i0, axis=1)
    hi = np.take_along_axis(s_dense, gidx + i1, axis=1)
    assert (p["s_codes"] == (lo | (hi << 4))).all()


def _decode_blocks(codes_dense, scale_bytes, blk, fmt):
    vals = e2m1_value(codes_dense)
    if fmt == oracle.MXFP4:
        sc = 2.0 ** (scale_bytes.astype(np.float64) - 127)
    else:
        sc = E4M3_VALUES[scale_bytes]
    return vals * np.repeat(sc, blk, axis=1)


def test_prepare_invariants_qkv():
    w = si.WORKLOADS["qkv_prefill"]
    x = si.workload_x(w, m=64)
    g = si.gamma(w.k, seed=11)                 # a non-unit gain too
    p = oracle.prepare(oracle.MXFP4, x, g, dense_backbone=True)
    xn_bits = oracle.normalize(x, g)
    xn = si.bf16_bits_to_f32(xn_bits).astype(np.float64)
    k = w.k
    nib = _unpack_meta(p["meta"], k)
    assert set(np.unique(nib)) <= {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}
    # exactly two kept per group, kept magnitudes >= dropped ones
    keep = np.zeros((64, k), bool)
    gidx = np.arange(k // 4) * 4
    np.put_along_axis(keep, gidx + (nib & 3), True, axis=1)
    np.put_along_axis(keep, gidx + (nib >> 2), True, axis=1)
    assert (keep.reshape(64, -1, 4).sum(-1) == 2).all()
    a = np.abs(xn).reshape(64, -1, 4)
    kk = keep.reshape(64, -1, 4)
    assert (np.where(kk, a, np.inf).min(-1) >= np.where(kk, -np.inf, a).max(-1)).all()
    # outlier-dominated backbone: its block scale is the plain MXFP4 scale of x_n
    plain = oracle.quantize_weight(oracle.MXFP4, xn_bits)
    assert (p["s_scales"] == plain["scales"]).all()
    # residual is exact: deq(backbone) + R == x_n bit for bit
    ds = _decode_blocks(_unpack_dense(p["s_dense"]), p["s_scales"], 32, oracle.MXFP4)
    assert (ds[~keep] == 0).all()
    r = oracle.residual_f32(oracle.MXFP4, xn_bits).astype(np.float64)
    assert (ds + r == xn).all()
    # residual quantization error: |deq(Qr) - R| <= 2 * S_r
    dr = _decode_blocks(_unpack_dense(p["r_codes"]), p["r_scales"], 32, oracle.MXFP4)
    sr = np.repeat(2.0 ** (p["r_scales"].astype(np.float64) - 127), 32, axis=1)
    assert (np.abs(dr - r) <= 2 * sr).all()
    # the decomposition beats plain MXFP4 of x_n
    dplain = _decode_blocks(_unpack_dense(plain["codes"]), plain["scales"], 32, oracle.MXFP4)
    assert np.linalg.norm(ds + dr - xn) < 0.5 * np.linalg.norm(dplain - xn)


def test_prepare_degenerate_rows():
    k = 64
    x = np.zeros((3, k), np.float32)
    x[1, 7] = -1000.0                       # one outlier
    x[2] = -0.0
    xb = si.f32_to_bf16_bits(x)
    p = oracle.prepare(oracle.MXFP4, xb, None)
    assert (p["s_scales"][0] == 0).all() and (p["r_scales"][0] == 0).all()
    assert (p["r_codes"][0] == 0).all() and (p["s_codes"][0] == 0).all()
    # all -0 row: mask keeps (0,1) per group; kept -0 -> code 8; kept residual
    # -0 - (-0) = +0 -> code 0; dropped residual -0 - (+0) = -0 -> code 8
    assert (_unpack_meta(p["meta"], k)[2] == 0x4).all()
    assert (p["s_codes"][2] == 0x88).all()
    assert (p["r_codes"][2, 0::2] == 0x00).all() and (p["r_codes"][2, 1::2] == 0x88).all()
    # outlier row: 1000 = 1.953125 * 2^9 -> scale 2^7, t = 7.8125 saturates to
    # code 7 (6 * 128 = 768), so the residual carries -1000 + 768 = -232
    assert p["s_scales"][1, 0] == 7 + 127
    # group 1 (k = 4..7) keeps k = 4 (a zero, lowest index) and k = 7: the
    # code at i1 (-6, 0xF) sits in the high nibble
    assert _unpack_meta(p["meta"], k)[1, 1] == (0 | 3 << 2)
    assert p["s_codes"][1, 1] == 0xF0
    r = oracle.residual_f32(oracle.MXFP4, oracle.normalize(xb, None))
    assert r[1, 7] == -232.0


# ------------------------------------------------------------ NVFP4-style
def _brute_prepare_nv(xn_bits):
    xn = si.bf16_bits_to_f32(xn_bits)
    m, k = xn.shape
    amax_t = np.float32(np.abs(xn).max())
    s_t = np.float32(1.0) if amax_t == 0 else np.float32(amax_t / np.float32(2688.0))

    def block(v):
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

    s_dense = np.zeros((m, k), np.uint8)
    s_scale = np.zeros((m, k // 16), np.uint8)
    r_codes = np.zeros((m, k), np.uint8)
    r_scale = np.zeros((m, k // 16), np.uint8)
    for i in range(m):
        v = np.zeros(k, np.float32)
        for g in range(k // 4):
            i0, i1 = mask_pair_brute(xn[i, 4 * g:4 * g + 4])
            v[4 * g + i0] = xn[i, 4 * g + i0]
            v[4 * g + i1] = xn[i, 4 * g + i1]
        d = np.zeros(k, np.float32)
        for b in range(k // 16):
            c, sb, dq = block(v[16 * b:16 * b + 16])
            s_dense[i, 16 * b:16 * b + 16] = c
            s_scale[i, b] = sb
            d[16 * b:16 * b + 16] = dq
        r = (xn[i] - d).astype(np.float32)
        for b in range(k // 16):
            c, sb, _ = block(r[16 * b:16 * b + 16])
            r_codes[i, 16 * b:16 * b + 16] = c
            r_scale[i, b] = sb
    return s_t, s_dense, s_scale, r_codes, r_scale


def test_prepare_nv_vs_brute():
    w = si.WORKLOADS["nvfp4_prefill"]
    x = si.workload_x(w, m=3)
    g = si.workload_gamma(w)
    p = oracle.prepare(oracle.NVFP4, x, g, dense_backbone=True)
    s_t, s_dense, s_scale, r_codes, r_scale = _brute_prepare_nv(oracle.normalize(x, g))
    assert p["tensor_scale"][0] == s_t
    assert (_unpack_dense(p["s_dense"]) == s_dense).all()
    assert (p["s_scales"] == s_scale).all()
    assert (_unpack_dense(p["r_codes"]) == r_codes).all()
    assert (p["r_scales"] == r_scale).all()


def test_nv_tensor_scale():
    assert oracle.nv_tensor_scale(0.0) == 1.0
    assert oracle.nv_tensor_scale(2688.0) == 1.0
    assert oracle.nv_tensor_scale(448.0 * 6 * 4) == 4.0


# ------------------------------------------------------------ weights
def test_quantize_weight_mx_vs_brute():
    w = si.weights(5, 256, seed=3)
    q = oracle.quantize_weight(oracle.MXFP4, w)
    wf = si.bf16_bits_to_f32(w).astype(np.float64)
    codes = _unpack_dense(q["codes"])
    for i in range(5):
        for b in range(8):
            c, sb, _ = mx_quantize_brute(wf[i, 32 * b:32 * b + 32])
            assert (codes[i, 32 * b:32 * b + 32] == c).all()
            assert q["scales"][i, b] == sb


def test_quantize_weight_nv_tensor_scale():
    w = si.weights(7, 64, seed=4)
    q = oracle.quantize_weight(oracle.NVFP4, w)
    amax = np.abs(si.bf16_bits_to_f32(w)).max()
    assert q["tensor_scale"][0] == np.float32(amax / np.float32(2688.0))


# ------------------------------------------------------------ GEMM
def test_dual_gemm_exact_rationals_tiny():
    w = si.WORKLOADS["tiny"]
    x = si.workload_x(w)
    W = si.workload_w(w)
    p = oracle.prepare(oracle.MXFP4, x, si.workload_gamma(w), dense_backbone=True)
    q = oracle.quantize_weight(oracle.MXFP4, W)
    rows = np.array([0, 3, 15], np.int64).repeat(4)
    cols = np.array([0, 77, 128, 255] * 3, np.int64)
    y, y64 = oracle.dual_gemm_pairs(oracle.MXFP4, p, q, rows, cols, want_f64=True)
    ds = _decode_blocks(_unpack_dense(p["s_dense"]), p["s_scales"], 32, oracle.MXFP4)
    dr = _decode_blocks(_unpack_dense(p["r_codes"]), p["r_scales"], 32, oracle.MXFP4)
    dw = _decode_blocks(_unpack_dense(q["codes"]), q["scales"], 32, oracle.MXFP4)
    for t, (i, j) in enumerate(zip(rows, cols)):
        exact = fraction_dot(ds[i], dw[j]) + fraction_dot(dr[i], dw[j])
        assert y64[t] == float(exact)
        assert y[t] == np.float32(y64[t])


def test_dual_gemm_matches_numpy_matmul():
    w = si.WORKLOADS["tiny"]
    x = si.workload_x(w)
    p = oracle.prepare(oracle.MXFP4, x, si.workload_gamma(w), dense_backbone=True)
    q = oracle.quantize_weight(oracle.MXFP4, si.workload_w(w))
    y = oracle.dual_gemm(oracle.MXFP4, p, q)
    ds = _decode_blocks(_unpack_dense(p["s_dense"]), p["s_scales"], 32, oracle.MXFP4)
    dr = _decode_blocks(_unpack_dense(p["r_codes"]), p["r_scales"], 32, oracle.MXFP4)
    dw = _decode_blocks(_unpack_dense(q["codes"]), q["scales"], 32, oracle.MXFP4)
    ref = ds @ dw.T + dr @ dw.T
    assert np.abs(y - ref).max() <= 1e-6 * np.abs(ref).max()
    # the pairs entry point agrees with the full one
    rows = np.repeat(np.arange(16), 3)
    cols = np.tile([1, 100, 200], 16)
    assert (oracle.dual_gemm_pairs(oracle.MXFP4, p, q, rows, cols) == y[rows, cols]).all()


def test_dual_gemm_nv_matches_numpy():
    x = si.activations("student_t4", 8, 128, 2, 50.0, 21)
    W = si.weights(24, 128, seed=22)
    p = oracle.prepare(oracle.NVFP4, x, si.gamma(128, None), dense_backbone=True)
    q = oracle.quantize_weight(oracle.NVFP4, W)
    y = oracle.dual_gemm(oracle.NVFP4, p, q)
    ds = _decode_blocks(_unpack_dense(p["s_dense"]), p["s_scales"], 16, oracle.NVFP4)
    dr = _decode_blocks(_unpack_dense(p["r_codes"]), p["r_scales"], 16, oracle.NVFP4)
    dw = _decode_blocks(_unpack_dense(q["codes"]), q["scales"], 16, oracle.NVFP4)
    ref = (ds @ dw.T + dr @ dw.T) * float(p["tensor_scale"][0]) * float(q["tensor_scale"][0])
    assert np.abs(y - ref).max() <= 1e-6 * np.abs(ref).max()


def test_special_case_exact_sparse_fp4_input():
    """X that is already 2:4 sparse and FP4-representable (any FP4 block keeps
    its values exactly under the OCP floor scale) is reproduced by the
    backbone: R = 0, the residual's codes and scale bytes are 0, and Y is the
    exact product rounded once."""
    rng = np.random.default_rng(5)
    m, k, n = 8, 256, 16
    x = e2m1_value(rng.integers(0, 16, (m, k)))
    for i in range(m):
        for g in range(k // 4):
            x[i, 4 * g + rng.choice(4, 2, replace=False)] = 0.0
    x = np.where(x == 0, 0.0, x) * 2.0 ** rng.integers(-3, 3, (m, 1))
    assert ((x.reshape(m, -1, 4) != 0).sum(-1) <= 2).all()
    xb = si.f32_to_bf16_bits(x.astype(np.float32))
    p = oracle.prepare(oracle.MXFP4, xb, None)
    assert (p["r_codes"] == 0).all() and (p["r_scales"] == 0).all()
    wv = e2m1_value(rng.integers(0, 16, (n, k))) * 2.0 ** rng.integers(-8, -4, (n, 1))
    wb = si.f32_to_bf16_bits(wv.astype(np.float32))
    q = oracle.quantize_weight(oracle.MXFP4, wb)
    y = oracle.dual_gemm(oracle.MXFP4, p, q)
    assert (y == (x @ wv.T).astype(np.float32)).all()


# ------------------------------------------------------------ grouped dual GEMM
def test_grouped_dual_gemm_one_group_is_dual_gemm():
    """One group with the identity gather is the plain dual GEMM, bit for bit."""
    w = si.WORKLOADS["tiny"]
    p = oracle.prepare(oracle.MXFP4, si.workload_x(w), si.workload_gamma(w))
    q = oracle.quantize_weight(oracle.MXFP4, si.workload_w(w))
    y = oracle.grouped_dual_gemm(oracle.MXFP4, p, None, [0, w.m], q, w.n)
    assert np.array_equal(y, oracle.dual_gemm(oracle.MXFP4, p, q))


def test_grouped_dual_gemm_rows_match_exact_products():
    """Each grouped row equals the exact dot products (rationals) of its
    gathered activation row with its group's weight rows; empty groups and a
    row used by two groups included."""
    rng = np.random.default_rng(5)
    t, k, n, groups = 9, 128, 6, 4
    x = si.activations("normal", t, k, 2, 8.0, 51)
    p = oracle.prepare(oracle.MXFP4, x, None, dense_backbone=True)
    q = oracle.quantize_weight(oracle.MXFP4, si.weights(groups * n, k, 52))
    offsets = [0, 3, 3, 8, 11]
    row_index = rng.integers(0, t, 11)
    row_index[4] = row_index[9] = 2
    y = oracle.grouped_dual_gemm(oracle.MXFP4, p, row_index, offsets, q, n)
    ds = _decode_blocks(_unpack_dense(p["s_dense"]), p["s_scales"], 32, oracle.MXFP4)
    dr = _decode_blocks(_unpack_dense(p["r_codes"]), p["r_scales"], 32, oracle.MXFP4)
    dw = _decode_blocks(_unpack_dense(q["codes"]), q["scales"], 32, oracle.MXFP4)
    for e in range(groups):
        for i in range(offsets[e], offsets[e + 1]):
            r = int(row_index[i])
            for j in range(n):
                exact = fraction_dot(ds[r], dw[e * n + j]) + fraction_dot(dr[r], dw[e * n + j])
                assert y[i, j] == np.float32(float(exact)), (e, i, j)


# ------------------------------------------------------------ gate+up GEMM, SiLU and the preparation
def test_dual_gemm_silu_prepare_vs_exact_product_and_decimal():
    """On FP4-grid inputs the preparation and the weight quantization keep
    every value exactly, so the dual GEMM is the exact product X W^T (numpy
    float64, exact for these values; fp32 holds it).  Then x[r, j] must be
    bf16(silu(Y[r, j]) * Y[r, inter + j]) by 60-digit Decimal arithmetic: the
    first inter rows of W are the gate, the last inter the up projection.  The
    returned operands dequantize to x within 2 2^e_r per block (e_r the
    residual's scale exponent: the E2M1 grid's widest gap is 2 at the top,
    and values up to 8 2^e_r saturate to 6 2^e_r)."""
    import decimal
    decimal.getcontext().prec = 60
    m, inter, k = 5, 128, 256
    xb = si.fp4_grid(m, k, 0, 61)
    wb = si.fp4_grid(2 * inter, k, -6, 62)
    X = si.bf16_bits_to_f32(xb).astype(np.float64)
    W = si.bf16_bits_to_f32(wb).astype(np.float64)
    p = oracle.prepare(oracle.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(oracle.MXFP4, wb)
    x, out = oracle.dual_gemm_silu_prepare(oracle.MXFP4, p, q, dense_backbone=True)
    Y = X @ W.T
    assert (Y.astype(np.float32).astype(np.float64) == Y).all()
    one = decimal.Decimal(1)
    for r in range(m):
        for j in range(0, inter, 5):
            g, u = decimal.Decimal(float(Y[r, j])), decimal.Decimal(float(Y[r, inter + j]))
            assert x[r, j] == _bf16_of_decimal(g / (one + (-g).exp()) * u), (r, j)
    # swapping the halves gives other values (the pin above tells them apart)
    assert (oracle.silu_mul(Y[:, inter:].astype(np.float32), Y[:, :inter].astype(np.float32)) != x).any()
    xf = si.bf16_bits_to_f32(x).astype(np.float64)
    ds = _decode_blocks(_unpack_dense(out["s_dense"]), out["s_scales"], 32, oracle.MXFP4)
    dr = _decode_blocks(_unpack_dense(out["r_codes"]), out["r_scales"], 32, oracle.MXFP4)
    bound = 2.0 * 2.0 ** (out["r_scales"].astype(np.float64) - 127)
    assert (np.abs(ds + dr - xf) <= np.repeat(bound, 32, axis=1)).all()


def test_grouped_dual_gemm_silu_prepare_rows_are_per_group_products():
    """Each grouped row of the grouped gate+up with SiLU is the single-row
    dual GEMM of its gathered activation row with its group's 2 inter weight
    rows (gate, then up), then SiLU(gate) * up and the preparation: checked
    against the plain (ungrouped) composition, which the pin above ties to the
    exact product and Decimal arithmetic; an empty group included."""
    inter, k, groups, t = 128, 256, 3, 7
    xb = si.fp4_grid(t, k, 0, 141)
    wb = si.fp4_grid(groups * 2 * inter, k, -6, 142)
    p = oracle.prepare(oracle.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(oracle.MXFP4, wb)
    offsets = [0, 4, 4, 9]
    row_index = np.array([6, 0, 3, 3, 1, 2, 5, 6, 0])
    x, out = oracle.grouped_dual_gemm_silu_prepare(oracle.MXFP4, p, row_index, offsets, q, inter, True)
    for e in range(groups):
        for i in range(offsets[e], offsets[e + 1]):
            xr, ref = oracle.dual_gemm_silu_prepare(oracle.MXFP4, oracle.gather_rows(p, [row_index[i]]),
                                                    oracle.expert_rows(q, e, 2 * inter), True)
            assert np.array_equal(x[i], xr[0]), (e, i)
            for key in ("s_codes", "meta", "s_scales", "s_dense", "r_codes", "r_scales"):
                assert np.array_equal(out[key][i], ref[key][0]), (e, i, key)
