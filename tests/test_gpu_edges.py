"""Every branch of the FP4 conversions, through the product kernels (needs an
MI355X), byte for byte against the oracle.

* The MXFP4 weight quantizer (gfx950's scaled bf16 -> FP4 conversion) on
  blocks that force every E8M0 byte a bf16 block can reach (0 .. 252) and
  carry every finite bf16 pattern at or below the block's maximum.
* The preparation without a norm, whose residual blocks take every E8M0 byte
  and hold every finite bf16 pattern (the fp32 -> FP4 conversion of the
  residual; abstract sentences 3-4 of arXiv:2606.26587).
* The NVFP4-style quantizer (sentence 7): exact E2M1 ties at power-of-two
  tensor scales, elements whose quotient lies within two ulps of a midpoint
  or whose code a reciprocal multiply would change, all-zero 16-blocks
  (S = 0), a tensor so small that S < 2^-100 (the kernels' IEEE division
  branch), one so large that S > 2^100, and blocks at the saturating ratio.
"""
import numpy as np
import pytest

import edge_inputs as ei
import oracle
import synth_inputs as si

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsity_fp4_quantized_amd as sq  # noqa: E402

DEV = "cuda:0"


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _same(label, got, want):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{label}: {len(bad)} bytes differ; first at {i}: gpu {got[i]:#04x} oracle {want[i]:#04x}")


def _check_weight(fmt, w, label, layout=sq.LAYOUT_KSTEP_MAJOR):
    ref = oracle.quantize_weight(fmt, w)
    q = sq.quantize_weight(dev16(w), fmt=fmt, layout=layout)
    _same(f"{label} codes", host(q.row_major("codes")), ref["codes"])
    _same(f"{label} scales", host(q.row_major("scales")), ref["scales"])
    if fmt == sq.NVFP4:
        assert host(q.tensor_scale)[0] == ref["tensor_scale"][0], label
    return ref


def _check_prep(fmt, x, label, gamma=None, layout=sq.LAYOUT_KSTEP_MAJOR):
    ref = oracle.prepare(fmt, x, gamma, 1e-5, dense_backbone=True)
    sp, rs = sq.prepare(dev16(x), None if gamma is None else dev16(gamma), 1e-5, fmt=fmt,
                        dense_backbone=True, layout=layout)
    for key, t in [("meta", sp.row_major("meta")), ("s_codes", sp.row_major("codes")),
                   ("s_scales", sp.row_major("scales")), ("s_dense", sp.row_major("dense_codes")),
                   ("r_codes", rs.row_major("codes")), ("r_scales", rs.row_major("scales"))]:
        _same(f"{label} {key}", host(t), ref[key])
    if fmt == sq.NVFP4:
        assert host(sp.tensor_scale)[0] == ref["tensor_scale"][0], label
    return ref


# ------------------------------------------------------------ MXFP4
@pytest.mark.parametrize("layout", [sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR])
def test_weight_mx_every_scale_byte_every_bf16(layout):
    w = ei.exhaustive_weight_mx(4096, seed=1)
    ref = _check_weight(sq.MXFP4, w, f"exhaustive weight {layout}", layout)
    assert (np.bincount(ref["scales"].ravel(), minlength=256)[:253] > 0).all()


def test_prepare_mx_residual_every_scale_byte_every_bf16():
    x = ei.exhaustive_residual_mx(4096, seed=2)
    ref = _check_prep(sq.MXFP4, x, "exhaustive residual")
    assert (np.bincount(ref["r_scales"].ravel(), minlength=256)[:253] > 0).all()


# ------------------------------------------------------------ NVFP4-style
@pytest.mark.parametrize("j", [-12, -3, 0, 4, 9])
def test_nv_weight_exact_ties(j):
    _check_weight(sq.NVFP4, ei.nv_tie_weight(j, seed=j + 20), f"nv ties 2^{j}")


def test_nv_prepare_exact_ties():
    # the same blocks as activations (no norm): kept values go through the
    # backbone's quantizer, dropped ones through the residual's
    _check_prep(sq.NVFP4, ei.nv_tie_weight(-2, seed=3), "nv prepare ties")


def test_nv_weight_near_midpoint_quotients():
    tensors = ei.nv_near_midpoint_weights(12, seed=4)
    for i, w in enumerate(tensors):
        _check_weight(sq.NVFP4, w, f"nv near-midpoint tensor {i}")
    for i, w in enumerate(tensors[:6]):
        _check_prep(sq.NVFP4, w, f"nv near-midpoint prepare {i}")


@pytest.mark.parametrize("kind", ["zero_blocks", "tiny", "huge", "saturate"])
def test_nv_degenerate_weights_and_prepare(kind):
    x = ei.nv_degenerate_rows(kind, m=12, k=256, seed=5)
    _check_weight(sq.NVFP4, x, f"nv weight {kind}")
    _check_prep(sq.NVFP4, x, f"nv prepare {kind}")
    if kind == "zero_blocks":
        _check_prep(sq.NVFP4, x, f"nv prepare {kind} norm", gamma=si.gamma(256, 6))
