"""Inputs built to reach every branch of the FP4 conversions (test side only).

The expected values always come from the oracle; these constructors only
arrange bf16 inputs so that every E8M0 block scale, every bf16 pattern below
a block's maximum, the NVFP4-style scale extremes and the E2M1 rounding ties
occur.  MXFP4 scale rule used to place the block maxima (OCP MX floor rule):
a block whose largest magnitude has binary exponent E gets scale exponent
E - 2, clamped to [-127, 127]; E8M0 byte = exponent + 127.
"""
from __future__ import annotations

import numpy as np

import synth_inputs as si
from brute import E4M3_VALUES, e2m1_argmin, e4m3_argmin

F32 = np.float32


def _bf16(v) -> np.ndarray:
    return si.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _bf16s(v) -> int:
    """bf16 bits of one value."""
    return int(_bf16(np.atleast_1d(np.float32(v))).ravel()[0])


def block_max_bits(e: int) -> int:
    """The largest positive bf16 whose block gets MX scale exponent e
    (-127 <= e <= 125): exponent field e + 129 with all mantissa bits set;
    for e = -127 every bf16 with exponent field <= 2 (subnormals included)."""
    field = 2 if e == -127 else e + 129
    assert 1 <= field <= 254
    return (field << 7) | 0x7F


def _rolled(blocks: np.ndarray, rng) -> np.ndarray:
    """Each row rotated by its own random amount (the block maximum lands on
    every lane position)."""
    n = blocks.shape[1]
    shift = rng.integers(0, n, blocks.shape[0])
    idx = (np.arange(n)[None, :] + shift[:, None]) % n
    return np.take_along_axis(blocks, idx, axis=1)


def _rows_of(blocks: np.ndarray, k: int) -> np.ndarray:
    """Blocks [nb, b] laid out as rows of k elements (zero blocks pad the last row)."""
    b = blocks.shape[1]
    per_row = k // b
    rows = -(-blocks.shape[0] // per_row)
    pad = rows * per_row - blocks.shape[0]
    if pad:
        blocks = np.concatenate([blocks, np.zeros((pad, b), blocks.dtype)])
    return blocks.reshape(rows, k)


def exhaustive_weight_mx(k: int = 4096, seed: int = 0) -> np.ndarray:
    """W [rows, k] (bf16 bits): for every MX scale byte a bf16 block can reach
    (0 .. 252), blocks whose maximum forces that byte and whose other 31
    entries run through every finite bf16 pattern (both signs) at or below
    that maximum.  Bytes 253 and 254 need a block maximum of 2^128 or more,
    beyond bf16."""
    rng = np.random.default_rng(seed)
    blocks = []
    for e in range(-127, 126):
        top = block_max_bits(e)
        pos = np.arange(0, top + 1, dtype=np.uint16)
        vals = np.concatenate([pos, pos | np.uint16(0x8000)])
        rng.shuffle(vals)
        nb = -(-vals.size // 31)
        body = np.zeros(nb * 31, np.uint16)
        body[:vals.size] = vals
        amax = np.full((nb, 1), top, np.uint16) | np.where(rng.random((nb, 1)) < 0.5, 0x8000, 0).astype(np.uint16)
        blocks.append(_rolled(np.concatenate([amax, body.reshape(nb, 31)], axis=1), rng))
    return _rows_of(np.concatenate(blocks), k)


def exhaustive_residual_mx(k: int = 4096, seed: int = 0, stride: int = 1) -> np.ndarray:
    """X [rows, k] (bf16 bits) for the preparation without a norm, built so
    that the RESIDUAL blocks take every MX scale byte 0 .. 252 and carry every
    finite bf16 pattern at or below their maximum (every `stride`-th pattern
    when stride > 1).  Each group of four holds two large values B = 6 2^es
    (es = er + 1; es = er = 125 at the top), exact at the backbone's scale,
    so the mask keeps them and the backbone reproduces them (residual 0
    there), and two test values below B, which the mask drops, so that the
    residual holds them exactly.  One test value per block is the residual
    block's maximum."""
    rng = np.random.default_rng(seed)
    out = []
    for er in range(-127, 126):
        es = er + 1 if er < 125 else 125
        bmag = F32(6.0 * 2.0 ** es)
        bbits = _bf16s(bmag)
        top = block_max_bits(er) if er < 125 else bbits          # residual block maximum
        top = min(top, bbits)
        pos = np.arange(0, top + 1, stride, dtype=np.uint16)
        vals = np.concatenate([pos, pos | np.uint16(0x8000)])
        rng.shuffle(vals)
        nb = -(-vals.size // 15)
        body = np.zeros(nb * 15, np.uint16)
        body[:vals.size] = vals
        tests = np.concatenate([np.full((nb, 1), top, np.uint16), body.reshape(nb, 15)], axis=1)
        tests = _rolled(tests, rng)                                # [nb, 16]: two per group
        big = np.full((nb, 16), bbits, np.uint16) | np.where(rng.random((nb, 16)) < 0.5, 0x8000, 0).astype(np.uint16)
        blk = np.empty((nb, 32), np.uint16)
        blk[:, 0::4], blk[:, 1::4] = big[:, 0::2], big[:, 1::2]
        blk[:, 2::4], blk[:, 3::4] = tests[:, 0::2], tests[:, 1::2]
        out.append(blk)
    return _rows_of(np.concatenate(out), k)


# ------------------------------------------------------------ NVFP4-style
MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def nv_tie_weight(j: int, seed: int = 0) -> np.ndarray:
    """W [rows, 128] (bf16 bits) whose tensor maximum is 2688 2^j, so the
    tensor scale is exactly 2^j; each 16-block has maximum e4m3(sb) 6 2^j for
    one sb and holds midpoint * S (S = e4m3(sb) 2^j, exact in bf16: the
    quotient lands on the E2M1 tie itself), their bf16 neighbours and signs."""
    rng = np.random.default_rng(seed)
    blocks = []
    for sb in range(1, 127):
        s = float(E4M3_VALUES[sb]) * 2.0 ** j
        ties = MIDPOINTS * s
        v = np.concatenate([ties, -ties])
        vb = _bf16(v)
        nb = np.concatenate([vb, vb + 1, vb - 1]).astype(np.uint16)      # next / previous bf16 of each
        nb = nb[((nb & 0x7F80) != 0) & ((nb & 0x7F80) != 0x7F80)]         # normal, finite
        cand = nb[np.abs(si.bf16_bits_to_f32(nb)) <= 6 * s]
        rng.shuffle(cand)
        for i in range(0, cand.size, 15):
            chunk = cand[i:i + 15]
            blk = np.zeros(16, np.uint16)
            blk[0] = _bf16s(6 * s)
            blk[1:1 + chunk.size] = chunk
            blocks.append(np.roll(blk, int(rng.integers(0, 16))))
    blocks.append(np.r_[np.uint16(_bf16s(2688.0 * 2.0 ** j)), np.zeros(15, np.uint16)])
    return _rows_of(np.array(blocks, np.uint16), 128)


def nv_near_midpoint_weights(count: int, seed: int = 0):
    """`count` weight tensors [rows, 128] (bf16 bits), each with its own
    tensor maximum A (tensor scale s_t = fl32(A / 2688)), holding elements v
    whose quotient fl32(v / S) lies within two ulps of an E2M1 midpoint or
    whose code differs from that of fl32(v * fl32(1 / S)): the cases where the
    element division must be the correctly rounded one."""
    rng = np.random.default_rng(seed)
    pos = np.arange(0x0080, 0x7F80, dtype=np.uint16)                 # positive normal bf16
    posf = si.bf16_bits_to_f32(pos)
    tensors = []
    while len(tensors) < count:
        A_bits = _bf16s(rng.uniform(0.5, 2.0) * 2.0 ** int(rng.integers(-30, 30)))
        A = F32(si.bf16_bits_to_f32(np.array([A_bits], np.uint16))[0])
        s_t = F32(A / F32(2688.0))
        d6 = F32(F32(6.0) * s_t)
        blocks = []
        for sb_want in range(1, 127):
            a_bits = _bf16s(F32(E4M3_VALUES[sb_want]) * d6)
            a = F32(si.bf16_bits_to_f32(np.array([a_bits], np.uint16))[0])
            if not (0 < a <= A):
                continue
            sb = int(e4m3_argmin(np.float64(F32(a / d6))))
            S = F32(F32(E4M3_VALUES[sb]) * s_t)
            if S == 0:
                continue
            sel = posf <= a
            v = posf[sel]
            t = (v / S).astype(np.float32)
            t_alt = (v * F32(F32(1.0) / S)).astype(np.float32)
            code = e2m1_argmin(t.astype(np.float64))
            near = np.zeros(v.size, bool)
            for m in MIDPOINTS:
                mb = np.float32(m).view(np.uint32).astype(np.int64)
                near |= np.abs(t.view(np.uint32).astype(np.int64) - mb) <= 2
            hit = near | (e2m1_argmin(t_alt.astype(np.float64)) != code)
            hv = pos[sel][hit]
            for i in range(0, hv.size, 15):
                chunk = hv[i:i + 15] | np.where(rng.random(min(15, hv.size - i)) < 0.5, 0x8000, 0).astype(np.uint16)
                blk = np.zeros(16, np.uint16)
                blk[0] = a_bits
                blk[1:1 + chunk.size] = chunk
                blocks.append(np.roll(blk, int(rng.integers(0, 16))))
        if not blocks:
            continue
        blocks.append(np.r_[np.uint16(A_bits), np.zeros(15, np.uint16)])
        tensors.append(_rows_of(np.array(blocks, np.uint16), 128))
    return tensors


def nv_degenerate_rows(kind: str, m: int = 12, k: int = 256, seed: int = 0) -> np.ndarray:
    """bf16 rows for the NVFP4-style edge branches:
      "zero_blocks": Student-t rows with whole 16-blocks of +0 and -0 (S = 0);
      "tiny": every value near 1e-38 (tensor scale subnormal, S < 2^-100);
      "huge": values near 3e38 (S > 2^100);
      "saturate": many blocks share the tensor maximum (ratio ~ 448)."""
    rng = np.random.default_rng(seed)
    if kind == "zero_blocks":
        x = rng.standard_t(4, (m, k)).astype(np.float32)
        for i in range(m):
            for b in rng.choice(k // 16, k // 64, replace=False):
                x[i, 16 * b:16 * b + 16] = -0.0 if (i + b) % 2 else 0.0
        return _bf16(x)
    if kind == "tiny":
        return _bf16(rng.standard_normal((m, k)) * 1e-38)
    if kind == "huge":
        return _bf16(rng.uniform(-1.0, 1.0, (m, k)) * 3.3e38)
    if kind == "saturate":
        x = rng.standard_normal((m, k)).astype(np.float32)
        x[:, ::16] = 40.0
        x[1::2, 5::16] = -40.0
        return _bf16(x)
    raise ValueError(kind)
