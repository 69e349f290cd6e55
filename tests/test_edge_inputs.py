"""The edge-case constructors reach what they claim (CPU, with the oracle):
every E8M0 byte 0 .. 252 with every finite bf16 pattern at or below the
block maximum, in the weight blocks and in the residual blocks of the
preparation; the NVFP4-style cases hit their branches."""
import numpy as np

import edge_inputs as ei
import oracle
import synth_inputs as si
from brute import E4M3_VALUES


def _coverage(values_bits: np.ndarray, scale_bytes: np.ndarray):
    """For each scale byte, the set of bf16 patterns seen in its blocks."""
    out = {}
    for s in np.unique(scale_bytes):
        out[int(s)] = np.unique(values_bits[scale_bytes == s])
    return out


def _expect_all_below(cov):
    for e in range(-127, 126):
        top = ei.block_max_bits(e)
        pos = np.arange(0, top + 1, dtype=np.uint16)
        want = np.union1d(pos, pos | np.uint16(0x8000))
        got = cov.get(e + 127)
        assert got is not None, e
        assert np.isin(want, got).all(), (e, int((~np.isin(want, got)).sum()))


def test_exhaustive_weight_covers_every_scale_and_pattern():
    w = ei.exhaustive_weight_mx(4096, seed=1)
    q = oracle.quantize_weight(oracle.MXFP4, w)
    blocks = w.reshape(-1, 32)
    sbytes = np.repeat(q["scales"].reshape(-1), 32)
    _expect_all_below(_coverage(blocks.reshape(-1), sbytes))


def test_exhaustive_residual_covers_every_scale_and_pattern():
    x = ei.exhaustive_residual_mx(4096, seed=2)
    p = oracle.prepare(oracle.MXFP4, x, None)
    r = oracle.residual_f32(oracle.MXFP4, x)
    rb = si.f32_to_bf16_bits(r)
    assert np.array_equal(si.bf16_bits_to_f32(rb), r)          # every residual is a bf16 value
    sbytes = np.repeat(p["r_scales"].reshape(-1), 32)
    cov = _coverage(rb.reshape(-1), sbytes)
    for e in range(-127, 125):
        top = ei.block_max_bits(e)
        pos = np.arange(0, top + 1, dtype=np.uint16)
        want = np.union1d(pos, pos | np.uint16(0x8000))
        assert np.isin(want, cov[e + 127]).all(), e
    # at the top scale the large values bound the test values at 1.5 2^127
    top = int(si.f32_to_bf16_bits(np.array([6.0 * 2.0 ** 125], np.float32))[0])
    pos = np.arange(0, top + 1, dtype=np.uint16)
    assert np.isin(np.union1d(pos, pos | np.uint16(0x8000)), cov[252]).all()


def test_nv_edge_constructors_reach_their_branches():
    # ties: the tensor scale is exactly 2^j and many quotients are midpoints
    w = ei.nv_tie_weight(-3, seed=1)
    q = oracle.quantize_weight(oracle.NVFP4, w)
    assert q["tensor_scale"][0] == np.float32(2.0 ** -3)
    # near-midpoint tensors are non-empty and of distinct tensor scales
    ts = [oracle.quantize_weight(oracle.NVFP4, t)["tensor_scale"][0] for t in ei.nv_near_midpoint_weights(4, seed=4)]
    assert len(set(ts)) == 4
    # S = 0, S < 2^-100 and S > 2^100
    p = oracle.prepare(oracle.NVFP4, ei.nv_degenerate_rows("zero_blocks"), None)
    assert (p["s_scales"] == 0).any()
    for kind, lo, hi in [("tiny", 0.0, 2.0 ** -100), ("huge", 2.0 ** 100, np.inf)]:
        p = oracle.prepare(oracle.NVFP4, ei.nv_degenerate_rows(kind), None)
        S = E4M3_VALUES[p["s_scales"].ravel()] * float(p["tensor_scale"][0])
        assert ((S > lo) & (S < hi)).mean() > 0.9, kind
    p = oracle.prepare(oracle.NVFP4, ei.nv_degenerate_rows("saturate"), None)
    assert (p["s_scales"] == 0x7E).sum() >= 12
