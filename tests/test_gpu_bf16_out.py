"""sharq_dual_gemm_bf16 (the dual GEMM with a bf16 output) on the GPU.

Three checks per case, every kernel the entry point dispatches to (prefill
128 x 128 and 128 x 192 dense-view tiles, 128 x 128 / 192 / 256 expanding
tiles, the skinny and decode kernels at m <= 32, the FP8 structured-sparse
variant, the NVFP4-style kernels):
  * bit for bit, the bf16 output equals the oracle's rounding (nearest even)
    of the fp32 output sharq_dual_gemm writes for the same inputs;
  * against the oracle, every output is the bf16 rounding of a value within
    the fp32 element-wise bound of the oracle's Y (tests/gemm_check.py);
  * on FP4-grid inputs, where the dual GEMM is exact in fp32, bit for bit
    the oracle's bf16 output.
Large shapes compare every 32-row and 32-column tile edge plus random
outputs with the oracle, and every output with the rounded fp32 result.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gemm_check import check_gemm_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsity_fp4_quantized_amd as sq  # noqa: E402
from test_gpu_parity import host, to_dev_prep, to_dev_weight  # noqa: E402

# (m, n, k, variant): the kernel each shape and variant takes
MX_CASES = [
    (300, 1000, 640, sq.GEMM_DENSE_EXPANDED),     # 128 x 128 dense-view tiles, ragged edges
    (2000, 6100, 384, sq.GEMM_DENSE_EXPANDED),    # 128 x 192 dense-view tiles
    (300, 1000, 640, sq.GEMM_DECOMPRESS),         # 128 x 128 expanding tiles
    (2000, 6100, 384, sq.GEMM_DECOMPRESS),        # 128 x 192 expanding tiles
    (2000, 4000, 640, sq.GEMM_DECOMPRESS),        # 128 x 256 expanding tiles
    (16, 1000, 640, sq.GEMM_DENSE_EXPANDED),      # skinny, dense view
    (7, 1000, 640, sq.GEMM_DECOMPRESS),           # skinny, 2:4 expanded in registers
    (16, 16500, 256, sq.GEMM_DENSE_EXPANDED),     # decode kernel
    (29, 16500, 256, sq.GEMM_DECOMPRESS),         # decode shape, 2:4 backbone
    (300, 1000, 640, sq.GEMM_SPARSE_MFMA),        # FP8 structured-sparse backbone
]
NV_VARIANTS = (sq.GEMM_DENSE_EXPANDED, sq.GEMM_DECOMPRESS, sq.GEMM_SPARSE_MFMA)


def sample(m, n, seed, count=4000):
    """Row, column pairs: every 32-row and 32-column tile edge, random outputs."""
    rng = np.random.default_rng(seed)
    er = np.concatenate([np.arange(0, m, 32), np.arange(31, m, 32), [m - 1]])
    ec = np.concatenate([np.arange(0, n, 32), np.arange(31, n, 32), [n - 1]])
    rows = np.concatenate([er, rng.integers(0, m, count), rng.integers(0, m, ec.size)])
    cols = np.concatenate([rng.integers(0, n, er.size), rng.integers(0, n, count), ec])
    order = np.argsort(rows, kind="stable")
    return rows[order], cols[order]


def both_outputs(fmt, p, q, variant, layout=sq.LAYOUT_KSTEP_MAJOR):
    sp, rs = to_dev_prep(fmt, p, layout)
    wq = to_dev_weight(fmt, q, layout)
    y32 = host(sq.dual_gemm(sp, rs, wq, variant=variant))
    y16 = host(sq.dual_gemm(sp, rs, wq, variant=variant, out_dtype=torch.bfloat16).view(torch.int16))
    return y32, y16.view(np.uint16)


def check_case(fmt, p, q, m, n, k, variant, label):
    y32, y16 = both_outputs(fmt, p, q, variant)
    assert y16.shape == (m, n)
    want = oracle.round_bf16(y32)
    if not np.array_equal(y16, want):
        i = tuple(np.argwhere(y16 != want)[0])
        raise AssertionError(f"{label}: {int((y16 != want).sum())} outputs differ from the rounded fp32 "
                             f"output; first at {i}: {y16[i]:#06x} against {want[i]:#06x} ({y32[i]!r})")
    if m * n <= 400_000:
        ref, yabs = oracle.dual_gemm_bound(fmt, p, q)
        check_gemm_bf16(y16, ref, yabs, k, label)
    else:
        rows, cols = sample(m, n, m + n + k)
        ref, yabs = oracle.dual_gemm_pairs_bound(fmt, p, q, rows, cols)
        check_gemm_bf16(y16[rows, cols], ref, yabs, k, label)


@pytest.mark.parametrize("m,n,k,variant", MX_CASES)
def test_dual_gemm_bf16_mx(m, n, k, variant):
    x = si.activations("student_t4", m, k, max(1, k // 100), 50.0, seed=m + 3 * n + k)
    w = si.weights(n, k, seed=m + n)
    p = oracle.prepare(sq.MXFP4, x, si.gamma(k, k), dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, w)
    check_case(sq.MXFP4, p, q, m, n, k, variant, f"mx m{m} n{n} k{k} v{variant}")


@pytest.mark.parametrize("m,n,k,variant", MX_CASES)
def test_dual_gemm_bf16_mx_exact(m, n, k, variant):
    """FP4-grid inputs: Y is exact in fp32 whatever the summation order, so
    the bf16 output must be the oracle's bit for bit."""
    xb = si.fp4_grid(m, k, 0, m + k)
    wb = si.fp4_grid(n, k, -6, n + k)
    p = oracle.prepare(sq.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    _, y16 = both_outputs(sq.MXFP4, p, q, variant)
    if m * n <= 400_000:
        want = oracle.dual_gemm_bf16(sq.MXFP4, p, q)
        got = y16
    else:
        rows, cols = sample(m, n, 7 * m + n)
        want = oracle.round_bf16(oracle.dual_gemm_pairs(sq.MXFP4, p, q, rows, cols))
        got = y16[rows, cols]
    assert np.array_equal(got, want), (m, n, k, variant, int((got != want).sum()))


@pytest.mark.parametrize("m,n,k", [(257, 300, 512), (16, 200, 256)])
@pytest.mark.parametrize("variant", NV_VARIANTS)
def test_dual_gemm_bf16_nv(m, n, k, variant):
    x = si.activations("student_t4", m, k, max(1, k // 100), 50.0, seed=5 * m + n)
    w = si.weights(n, k, seed=n + k)
    p = oracle.prepare(sq.NVFP4, x, si.gamma(k, 3), dense_backbone=True)
    q = oracle.quantize_weight(sq.NVFP4, w)
    check_case(sq.NVFP4, p, q, m, n, k, variant, f"nv m{m} n{n} k{k} v{variant}")


def test_dual_gemm_bf16_row_major_and_padded_output():
    """Row-major operands and a bf16 output with a padded row stride: the
    padding is left untouched and the values equal the contiguous output's."""
    m, n, k = 200, 390, 384
    x = si.activations("student_t4", m, k, 4, 50.0, seed=71)
    p = oracle.prepare(sq.MXFP4, x, si.gamma(k, 72), dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, si.weights(n, k, seed=73))
    sp, rs = to_dev_prep(sq.MXFP4, p, sq.LAYOUT_ROW_MAJOR)
    wq = to_dev_weight(sq.MXFP4, q, sq.LAYOUT_ROW_MAJOR)
    ref16 = sq.dual_gemm(sp, rs, wq, out_dtype=torch.bfloat16)
    big = torch.full((m, n + 40), -7.0, dtype=torch.bfloat16, device="cuda:0")
    out = big[:, :n]
    sq.dual_gemm(sp, rs, wq, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref16.view(torch.int16))
    assert bool((big[:, n:] == -7.0).all())
    y32 = host(sq.dual_gemm(sp, rs, wq))
    assert np.array_equal(host(ref16.view(torch.int16)).view(np.uint16), oracle.round_bf16(y32))
