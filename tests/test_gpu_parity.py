"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Masks, FP4 codes and scales must be byte-identical; GEMM outputs must be
within 1e-3 of the oracle's, normwise (max |dY| / max |Y|), the bound the
SharQ path is built to, and every output within 4 K 2^-24 of the sum of the
magnitudes of its products (tests/gemm_check.py); where the product is exact
in fp32 the GEMM must match bit for bit.  Every call goes through the C ABI in
include/sharq.h.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gemm_check import check_gemm

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparsity_fp4_quantized_amd as sq  # noqa: E402

DEV = "cuda:0"


def dev16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_prep(fmt, x_bits, gamma_bits, eps=1e-5, dense=True, label="", layout=None):
    ref = oracle.prepare(fmt, x_bits, gamma_bits, eps, dense_backbone=True)
    sp, rs = sq.prepare(dev16(x_bits), None if gamma_bits is None else dev16(gamma_bits), eps,
                        fmt=fmt, dense_backbone=dense, layout=layout)
    got = {"meta": host(sp.row_major("meta")), "s_codes": host(sp.row_major("codes")),
           "s_scales": host(sp.row_major("scales")),
           "r_codes": host(rs.row_major("codes")), "r_scales": host(rs.row_major("scales"))}
    if dense:
        got["s_dense"] = host(sp.row_major("dense_codes"))
    for key, val in got.items():
        want = ref[key]
        if not np.array_equal(val, want):
            bad = np.argwhere(val != want)
            r, c = bad[0]
            raise AssertionError(f"{label} {key}: {len(bad)} bytes differ; first at row {r} col {c}: "
                                 f"gpu {val[r, c]:#04x} oracle {want[r, c]:#04x}")
    if fmt == sq.NVFP4:
        ts = host(sp.tensor_scale)
        assert ts[0] == ref["tensor_scale"][0], (label, ts, ref["tensor_scale"])
    return ref, sp, rs


def to_layout(rowmajor: np.ndarray, bps: int, layout):
    """Row-major [rows, steps * bps] array as a device array in `layout`."""
    if layout == sq.LAYOUT_KSTEP_MAJOR:
        rows, nb = rowmajor.shape
        rowmajor = rowmajor.reshape(rows, nb // bps, bps).transpose(1, 0, 2)
    return torch.from_numpy(np.ascontiguousarray(rowmajor)).to(DEV)


def dev_scales(rowmajor: np.ndarray, fmt, layout):
    return to_layout(rowmajor, sq.scale_bps(fmt), layout)


def to_dev_weight(fmt, q, layout=sq.LAYOUT_KSTEP_MAJOR):
    n, kh = q["codes"].shape
    w = sq.FP4Tensor(fmt, n, kh * 2, to_layout(q["codes"], sq.BPS_CODES, layout),
                     dev_scales(q["scales"], fmt, layout), layout=layout)
    if fmt == sq.NVFP4:
        w.tensor_scale = torch.tensor([q["tensor_scale"][0], 0.0], dtype=torch.float32, device=DEV)
    return w


def to_dev_prep(fmt, p, layout=sq.LAYOUT_KSTEP_MAJOR):
    """Oracle preparation outputs as device FP4 tensors (GEMM-only tests)."""
    m, kq = p["s_codes"].shape
    k = kq * 4
    sp = sq.FP4Tensor(fmt, m, k, to_layout(p["s_codes"], sq.BPS_SPARSE_CODES, layout),
                      dev_scales(p["s_scales"], fmt, layout),
                      meta=to_layout(p["meta"], sq.BPS_META, layout), layout=layout)
    if "s_dense" in p:
        sp.dense_codes = to_layout(p["s_dense"], sq.BPS_CODES, layout)
    rs = sq.FP4Tensor(fmt, m, k, to_layout(p["r_codes"], sq.BPS_CODES, layout),
                      dev_scales(p["r_scales"], fmt, layout), layout=layout)
    if fmt == sq.NVFP4:
        ts = torch.tensor([p["tensor_scale"][0], 0.0], dtype=torch.float32, device=DEV)
        sp.tensor_scale = ts
        rs.tensor_scale = ts
    return sp, rs


# ------------------------------------------------------------ preparation
@pytest.mark.parametrize("m,k,norm", [
    (1, 32, True), (5, 96, True), (7, 256, True), (37, 1024, True), (4, 4096, True),
    (3, 14336, True), (9, 16384, True), (6, 32, False), (13, 14336, False), (2, 65536, False),
])
def test_prepare_mx_shapes(m, k, norm):
    x = si.activations("student_t4", m, k, max(1, k // 100), 50.0, seed=m * 1000 + k)
    g = si.gamma(k, seed=k) if norm else None
    check_prep(sq.MXFP4, x, g, label=f"m{m} k{k} norm{norm}")


@pytest.mark.parametrize("name", ["tiny", "qkv_prefill", "down_prefill", "decode_gate_up"])
def test_prepare_mx_workloads(name):
    w = si.WORKLOADS[name]
    check_prep(sq.MXFP4, si.workload_x(w), si.workload_gamma(w), label=name)


@pytest.mark.parametrize("fmt,norm", [(0, True), (0, False), (1, True), (1, False)])
def test_prepare_layouts(fmt, norm):
    """Both layouts hold the same bytes."""
    x = si.activations("student_t4", 21, 512, 5, 50.0, seed=44 + fmt)
    g = si.gamma(512, 6) if norm else None
    for layout in (sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR):
        check_prep(fmt, x, g, label=f"layout {layout}", layout=layout)


@pytest.mark.parametrize("m,k", [(1030, 4096), (600, 2048), (530, 8192), (1027, 8192)])
def test_prepare_mx_row_groups(m, k):
    """Row counts that take the normalized preparation's 4- and 2-row
    wavefront groups (ragged last group), in both layouts."""
    x = si.activations("student_t4", m, k, max(1, k // 100), 50.0, seed=m + k)
    g = si.gamma(k, seed=k + 1)
    for layout in (sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR):
        check_prep(sq.MXFP4, x, g, label=f"m{m} k{k} layout {layout}", layout=layout)


def test_prepare_mx_degenerate_rows():
    k = 256
    x = np.zeros((6, k), np.float32)
    x[1, 7] = -1000.0                 # a single outlier
    x[2] = -0.0                       # signed zeros
    x[3] = 1.0                        # all ties
    x[4, ::3] = 3e-39                 # fp32-subnormal squares underflow
    x[5] = np.tile([2.0, -2.0, 2.0, 1.0], k // 4)
    xb = si.f32_to_bf16_bits(x)
    check_prep(sq.MXFP4, xb, None, label="degenerate no-norm")
    check_prep(sq.MXFP4, xb, si.gamma(k, None), label="degenerate norm")


@pytest.mark.parametrize("m,k", [(1, 32), (3, 96), (16, 224), (32, 512), (7, 992), (16, 4096),
                                 (29, 8192), (32, 6144)])
def test_prepare_mx_few_rows(m, k):
    """m <= 32 rows with the norm and k <= 8192 (decode): four lanes share a
    block (prep_norm_quad_kernel), one workgroup a row; random gain, both
    layouts where k allows, with and without the dense backbone view."""
    x = si.activations("student_t4", m, k, max(1, k // 100), 50.0, seed=3 * m + k)
    g = si.gamma(k, seed=k + 5)
    for layout in (sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR) if k % 128 == 0 else (None,):
        check_prep(sq.MXFP4, x, g, label=f"few rows m{m} k{k} layout {layout}", layout=layout)
    check_prep(sq.MXFP4, x, g, dense=False, label=f"few rows m{m} k{k} no dense view")


def test_prepare_mx_few_rows_match_row_groups():
    """The same rows prepared with 32 rows (four lanes a block) and 33 rows
    (one lane a block): identical bytes for the common rows."""
    k = 4096
    x = si.activations("student_t4", 33, k, 41, 50.0, seed=91)
    g = si.gamma(k, seed=92)
    sp33, rs33 = sq.prepare(dev16(x), dev16(g), 1e-5, dense_backbone=True)
    sp32, rs32 = sq.prepare(dev16(x[:32]), dev16(g), 1e-5, dense_backbone=True)
    for t33, t32, key in ((sp33, sp32, "codes"), (sp33, sp32, "meta"), (sp33, sp32, "scales"),
                          (sp33, sp32, "dense_codes"), (rs33, rs32, "codes"), (rs33, rs32, "scales")):
        assert np.array_equal(host(t33.row_major(key))[:32], host(t32.row_major(key))), key


@pytest.mark.parametrize("k", [224, 4000])
def test_prepare_mx_row_mean_ranges(k):
    """Finite rows whose sums of squares span 2^-130 .. Inf: the row mean's
    Markstein path (ss in [2^-100, 2^100] or 0), its IEEE-division path on
    both sides and a sum that overflows to Inf (r = 0, x_n = 0).  Inf and NaN
    elements are outside the supported inputs."""
    rows = []
    for e in range(-70, 71, 4):
        x = si.bf16_bits_to_f32(si.activations("student_t4", 1, k, 2, 50.0, seed=e + 100))[0]
        rows.append(x * np.float32(2.0 ** e))
    rows.append(np.zeros(k, np.float32))
    xb = si.f32_to_bf16_bits(np.stack(rows))
    for layout in (sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR) if k % 128 == 0 else (None,):
        check_prep(sq.MXFP4, xb, si.gamma(k, seed=3), label=f"row mean ranges k{k}", layout=layout)
        # at most 32 rows a call: the few-rows kernel (four lanes a block)
        for part in (xb[:32], xb[32:]):
            check_prep(sq.MXFP4, part, si.gamma(k, seed=3), label=f"row mean ranges few rows k{k}", layout=layout)


def test_prepare_padded_row_stride():
    m, k, ld = 10, 512, 640
    x = si.activations("normal", m, ld, 3, 40.0, seed=77)
    g = si.gamma(k, seed=5)
    xt = dev16(x)[:, :k]
    assert xt.stride(0) == ld
    ref = oracle.prepare(sq.MXFP4, np.ascontiguousarray(x[:, :k]), g)
    for layout in (sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR):
        sp, rs = sq.prepare(xt, dev16(g), 1e-5, layout=layout)
        assert np.array_equal(host(sp.row_major("codes")), ref["s_codes"])
        assert np.array_equal(host(rs.row_major("codes")), ref["r_codes"])
        assert np.array_equal(host(sp.row_major("meta")), ref["meta"])


@pytest.mark.parametrize("norm", [True, False])
def test_prepare_padded_row_stride_row_groups(norm):
    """Row strides above k with several rows per wavefront (four with the
    norm, sixteen in the k-step-major flat kernel), where each lane's offset
    in X carries its row within the group times the stride; both layouts."""
    m, k, ld = 1100, 1024, 1024 + 192
    x = si.activations("student_t4", m, ld, 12, 50.0, seed=78)
    g = si.gamma(k, seed=79) if norm else None
    xt = dev16(x)[:, :k]
    assert xt.stride(0) == ld
    ref = oracle.prepare(sq.MXFP4, np.ascontiguousarray(x[:, :k]), g, dense_backbone=True)
    for layout in (sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR):
        sp, rs = sq.prepare(xt, None if g is None else dev16(g), 1e-5, dense_backbone=True, layout=layout)
        _compare_prep(f"padded rows norm{norm} layout {layout}", sp, rs, ref)


def test_prepare_residual_padded_row_groups():
    """The residual add with padded h, o and x_out at four rows per
    wavefront: each input's own stride in every lane offset."""
    m, k = 1100, 2048
    h = si.activations("student_t4", m, k, 20, 50.0, seed=80)
    o = si.activations("normal", m, k, 0, 1.0, seed=81)
    g = si.gamma(k, 82)
    x_ref, ref = oracle.prepare_residual(sq.MXFP4, h, o, g, dense_backbone=True)
    hb = torch.zeros((m, k + 64), dtype=torch.int16, device=DEV)
    ob = torch.zeros((m, k + 128), dtype=torch.int16, device=DEV)
    xb = torch.full((m, k + 256), 0x7A5A, dtype=torch.int16, device=DEV)
    hb[:, :k] = dev16(h)
    ob[:, :k] = dev16(o)
    x, sp, rs = sq.prepare_residual(hb[:, :k], ob[:, :k], dev16(g), dense_backbone=True, out=xb[:, :k])
    got = host(xb).view(np.uint16)
    assert np.array_equal(got[:, :k], x_ref)
    assert (got[:, k:] == 0x7A5A).all()
    _compare_prep("residual padded row groups", sp, rs, ref)


def test_prepare_nv_small():
    for m, k, norm in [(3, 64, True), (17, 512, False), (8, 4096, True)]:
        x = si.activations("student_t4", m, k, 2, 50.0, seed=31 + k)
        check_prep(sq.NVFP4, x, si.gamma(k, 3) if norm else None, label=f"nv m{m} k{k}")


def test_prepare_nv_workload():
    w = si.WORKLOADS["nvfp4_prefill"]
    check_prep(sq.NVFP4, si.workload_x(w), si.workload_gamma(w), label="nvfp4_prefill")


def test_prepare_deterministic():
    w = si.WORKLOADS["qkv_prefill"]
    x = dev16(si.workload_x(w, m=512))
    g = dev16(si.workload_gamma(w))
    a = sq.prepare(x, g)
    b = sq.prepare(x, g)
    for t1, t2 in [(a[0].codes, b[0].codes), (a[0].meta, b[0].meta), (a[1].codes, b[1].codes)]:
        assert torch.equal(t1, t2)



def test_bound_calls_match_one_shot_calls():
    """bind_prepare / bind_dual_gemm (arguments marshalled once, as bench.py
    runs them) give the bytes of the one-shot calls, call after call, and
    write into the buffers they were bound to."""
    w = si.WORKLOADS["qkv_prefill"]
    x = dev16(si.workload_x(w, m=300))
    g = dev16(si.workload_gamma(w))
    wq = sq.quantize_weight(dev16(si.workload_w(w, n=200)))
    sp0, rs0 = sq.prepare(x, g, dense_backbone=True)
    y0 = sq.dual_gemm(sp0, rs0, wq)
    sp, rs = sq.alloc_prepared(sq.MXFP4, 300, w.k, DEV, dense_backbone=True)
    y = torch.full_like(y0, float("nan"))
    prep, gemm = sq.bind_prepare(x, g, 1e-5, sp, rs), sq.bind_dual_gemm(sp, rs, wq, y)
    for _ in range(3):
        prep()
        gemm()
        torch.cuda.synchronize()
        for t1, t2 in [(sp.codes, sp0.codes), (sp.meta, sp0.meta), (sp.scales, sp0.scales),
                       (sp.dense_codes, sp0.dense_codes), (rs.codes, rs0.codes), (rs.scales, rs0.scales)]:
            assert torch.equal(t1, t2)
        assert torch.equal(y, y0)
        y.fill_(float("nan"))



def _compare_prep(label, sp, rs, ref, dense=True):
    got = {"meta": host(sp.row_major("meta")), "s_codes": host(sp.row_major("codes")),
           "s_scales": host(sp.row_major("scales")),
           "r_codes": host(rs.row_major("codes")), "r_scales": host(rs.row_major("scales"))}
    if dense:
        got["s_dense"] = host(sp.row_major("dense_codes"))
    for key, val in got.items():
        assert np.array_equal(val, ref[key]), (label, key, int((val != ref[key]).sum()))


@pytest.mark.parametrize("m,k,where", [(2048, 4096, "new"), (600, 2048, "h"), (37, 4096, "o"),
                                       (1027, 8192, "new"), (5, 256, "h")])
def test_prepare_residual(m, k, where):
    """Residual add fused into the preparation: the new residual stream and
    every prepared array byte for byte against the oracle (four, two and one
    rows per wavefront; written to a new tensor, or in place on h or on o)."""
    h = si.activations("student_t4", m, k, 41 if k >= 4096 else 4, 50.0, seed=31)
    o = si.activations("normal", m, k, 0, 1.0, seed=32)
    g = si.gamma(k, 33)
    x_ref, ref = oracle.prepare_residual(sq.MXFP4, h, o, g, dense_backbone=True)
    dh, do = dev16(h), dev16(o)
    out = {"new": None, "h": dh, "o": do}[where]
    x, sp, rs = sq.prepare_residual(dh, do, dev16(g), dense_backbone=True, out=out)
    assert np.array_equal(host(x).view(np.uint16), x_ref), "residual stream"
    if where == "h":
        assert np.array_equal(host(dh).view(np.uint16), x_ref)
    _compare_prep(f"m{m} k{k} {where}", sp, rs, ref)


def test_prepare_residual_padded_rows_untouched():
    """Row strides above k: the padding of the output rows is never written."""
    m, k, ld = 300, 4096, 4096 + 64
    h = si.activations("student_t4", m, k, 41, 50.0, seed=34)
    o = si.activations("normal", m, k, 0, 1.0, seed=35)
    g = si.gamma(k, 36)
    x_ref, ref = oracle.prepare_residual(sq.MXFP4, h, o, g, dense_backbone=True)
    big = torch.full((m, ld), 0x7A5A, dtype=torch.int16, device=DEV)
    hb = torch.full((m, ld), 0, dtype=torch.int16, device=DEV)
    hb[:, :k] = dev16(h)
    x, sp, rs = sq.prepare_residual(hb[:, :k], dev16(o), dev16(g), dense_backbone=True, out=big[:, :k])
    got = host(big).view(np.uint16)
    assert np.array_equal(got[:, :k], x_ref)
    assert (got[:, k:] == 0x7A5A).all()
    _compare_prep("padded", sp, rs, ref)


def test_bound_prepare_residual_repeats():
    """bind_prepare_residual called again on its own output (a residual stream
    that keeps growing) matches the oracle step after step."""
    m, k = 64, 4096
    h = si.activations("student_t4", m, k, 41, 50.0, seed=37)
    o = si.activations("normal", m, k, 0, 1.0, seed=38)
    g = si.gamma(k, 39)
    dh = dev16(h)
    sp, rs = sq.alloc_prepared(sq.MXFP4, m, k, DEV, dense_backbone=True)
    call = sq.bind_prepare_residual(dh, dev16(o), dev16(g), 1e-5, sp, rs, dh)
    x = h
    for step in range(3):
        call()
        x, ref = oracle.prepare_residual(sq.MXFP4, x, o, g, dense_backbone=True)
        assert np.array_equal(host(dh).view(np.uint16), x), step
        _compare_prep(f"step {step}", sp, rs, ref)



@pytest.mark.parametrize("m,k,layout", [(2048, 14336, sq.LAYOUT_KSTEP_MAJOR), (16, 14336, sq.LAYOUT_KSTEP_MAJOR),
                                        (37, 4096, sq.LAYOUT_KSTEP_MAJOR), (37, 4096, sq.LAYOUT_ROW_MAJOR),
                                        (3, 96, sq.LAYOUT_ROW_MAJOR)])
def test_prepare_silu_mul(m, k, layout):
    """SiLU(gate) * up fused into the preparation, gate and up being the two
    column halves of one fp32 [m, 2k] gate+up output: every prepared array
    byte for byte against the oracle.  The inputs include gates outside the
    fp32 fast path (|g| > 64, tiny), signed zero gates against ups of both
    signs and signed zero ups (exact on the fast path), and zero ups."""
    g, u = si.gate_up_output(m, k, seed=41)
    g[0, :8] = [0.0, -0.0, 1e-30, -70.0, 90.0, -100.0, 65.0, -64.0]
    u[0, 8:12] = [0.0, -0.0, 0.0, 0.0]
    if m > 1:
        g[1, :8] = [0.0, -0.0, 0.0, -0.0, 0.0, -0.0, 0.0, -0.0]
        u[1, :8] = [1.5, 1.5, -2.5, -2.5, 0.0, 0.0, -0.0, -0.0]
    _, ref = oracle.prepare_silu_mul(sq.MXFP4, g, u, dense_backbone=True)
    gu = torch.from_numpy(np.concatenate([g, u], axis=1)).to(DEV)
    sp, rs = sq.prepare_silu_mul(gu[:, :k], gu[:, k:], dense_backbone=True, layout=layout)
    _compare_prep(f"silu m{m} k{k}", sp, rs, ref)



def test_prepare_silu_mul_top_binade():
    """silu(g) * u in the largest bf16 binade, [2^127, 3.39e38], through the
    binary64 path (|g| > 8), with neighbours that round down to the largest
    finite bf16: the rounding's overflow guard must leave these finite values
    alone.  Byte for byte against the oracle."""
    rng = np.random.default_rng(77)
    m, k = 8, 256
    g = rng.uniform(8.5, 1e4, (m, k)).astype(np.float32)
    target = rng.uniform(2.0 ** 127, 3.38e38, (m, k)) * np.where(rng.random((m, k)) < 0.5, -1, 1)
    gd = g.astype(np.float64)
    u = (target / (gd / (1.0 + np.exp(-gd)))).astype(np.float32)
    u[:, 1::4] *= np.float32(1e-3)          # smaller values in every group
    x, ref = oracle.prepare_silu_mul(sq.MXFP4, g, u, dense_backbone=True)
    assert ((x & 0x7F80) != 0x7F80).all() and ((x & 0x7F80) == 0x7F00).mean() > 0.5
    sp, rs = sq.prepare_silu_mul(torch.from_numpy(g).to(DEV), torch.from_numpy(u).to(DEV), dense_backbone=True)
    _compare_prep("silu top binade", sp, rs, ref)


def _grouped_case(tokens, k, n, experts, top_k, seed, layout=sq.LAYOUT_KSTEP_MAJOR):
    x = si.activations("student_t4", tokens, k, 41 if k >= 4096 else 20, 50.0, seed)
    g = si.gamma(k, seed + 1)
    W = si.weights(experts * n, k, seed + 2)
    row_index, offsets = si.moe_routing(tokens, experts, top_k, seed + 3)
    p = oracle.prepare(sq.MXFP4, x, g, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, W)
    sp, rs = sq.prepare(dev16(x), dev16(g), dense_backbone=True, layout=layout)
    wq = sq.quantize_weight(dev16(W), layout=layout)
    return p, q, sp, rs, wq, row_index, offsets


@pytest.mark.parametrize("tokens,k,n,experts,top_k,layout", [
    (300, 2048, 320, 8, 2, sq.LAYOUT_KSTEP_MAJOR),
    (200, 768, 256, 16, 4, sq.LAYOUT_KSTEP_MAJOR),
    (150, 256, 200, 5, 3, sq.LAYOUT_ROW_MAJOR),
    (4096, 256, 512, 32, 8, sq.LAYOUT_KSTEP_MAJOR),    # enough tiles for the 128 x 256 tiles
    (4096, 256, 384, 32, 8, sq.LAYOUT_KSTEP_MAJOR),    # 128 x 256, n ragged
    (4096, 256, 256, 32, 8, sq.LAYOUT_KSTEP_MAJOR),    # 128 x 192, n ragged
])
def test_grouped_dual_gemm(tokens, k, n, experts, top_k, layout):
    """Grouped (mixture-of-experts) dual GEMM over gathered activation rows
    against the oracle, every output: uneven groups (some over one 128-row
    tile, some of a few rows), both layouts."""
    p, q, sp, rs, wq, row_index, offsets = _grouped_case(tokens, k, n, experts, top_k, 61, layout)
    rows = int(offsets[-1])
    ref, yabs = oracle.grouped_dual_gemm_bound(sq.MXFP4, p, row_index, offsets, q, n)
    y = host(sq.grouped_dual_gemm(sp, rs, wq, torch.from_numpy(offsets).to(DEV), rows,
                                  row_index=torch.from_numpy(row_index).to(DEV)))
    check_gemm(y, ref, yabs, k, "test_grouped_dual_gemm")
    # each group's rows also equal the plain dual GEMM of the gathered rows
    e = int(np.argmax(np.diff(offsets)))
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    sub, subabs = oracle.dual_gemm_bound(sq.MXFP4, oracle.gather_rows(p, row_index[lo:hi]), oracle.expert_rows(q, e, n))
    check_gemm(y[lo:hi], sub, subabs, k, "test_grouped_dual_gemm group")


def test_grouped_dual_gemm_identity_gather_and_empty_groups():
    """row_index None (the rows already grouped), empty groups, one group
    holding everything: equal to the plain dual GEMM of each group's rows."""
    tokens, k, n = 260, 512, 192
    x = si.activations("student_t4", tokens, k, 20, 50.0, 71)
    W = si.weights(3 * n, k, 72)
    p = oracle.prepare(sq.MXFP4, x, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, W)
    sp, rs = sq.prepare(dev16(x), None, dense_backbone=True)
    wq = sq.quantize_weight(dev16(W))
    for offsets in ([0, 0, 260, 260], [0, 1, 129, 250]):
        offsets = np.array(offsets, np.int64)
        rows = int(offsets[-1])
        y = host(sq.grouped_dual_gemm(sp, rs, wq, torch.from_numpy(offsets).to(DEV), rows))
        ref, yabs = oracle.grouped_dual_gemm_bound(sq.MXFP4, p, None, offsets, q, n)
        check_gemm(y, ref, yabs, k, f"test_grouped_dual_gemm_identity_gather_and_empty_groups {offsets}")


# group sizes whose last 128-row tile ends in every 32-row quarter and on its
# edges: wavefronts with both, one or none of their 32-row tiles in the group
_RESIDUE_GROUPS = [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 161, 192, 255]


def test_grouped_dual_gemm_tile_residues():
    """Groups whose sizes end their last tile in every 32-row quarter (the
    tiles past a group's end skip their MFMAs and read zeros): every output
    against the oracle, through a random gather."""
    k, n = 256, 192
    sizes = np.array(_RESIDUE_GROUPS, np.int64)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    rows, tokens = int(offsets[-1]), 700
    x = si.activations("student_t4", tokens, k, 20, 50.0, 91)
    W = si.weights(len(sizes) * n, k, 92)
    row_index = np.random.default_rng(93).integers(0, tokens, rows).astype(np.int32)
    p = oracle.prepare(sq.MXFP4, x, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, W)
    sp, rs = sq.prepare(dev16(x), None, dense_backbone=True)
    wq = sq.quantize_weight(dev16(W))
    ref, yabs = oracle.grouped_dual_gemm_bound(sq.MXFP4, p, row_index, offsets, q, n)
    y = host(sq.grouped_dual_gemm(sp, rs, wq, torch.from_numpy(offsets).to(DEV), rows,
                                  row_index=torch.from_numpy(row_index).to(DEV)))
    check_gemm(y, ref, yabs, k, "test_grouped_dual_gemm_tile_residues")


def test_grouped_dual_gemm_silu_prepare_tile_residues():
    """The fused gate+up form on the same group sizes, FP4-grid inputs: every
    prepared byte of every grouped row against the oracle."""
    k, inter = 256, 128
    sizes = np.array(_RESIDUE_GROUPS, np.int64)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    rows, tokens = int(offsets[-1]), 700
    xb, wb, _, _, sp, rs, wq = _grouped_silu_grid_case(tokens, k, inter, len(sizes), 1, 131, KSM)
    row_index = np.random.default_rng(133).integers(0, tokens, rows).astype(np.int32)
    p = oracle.prepare(sq.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    _, ref = oracle.grouped_dual_gemm_silu_prepare(sq.MXFP4, p, row_index, offsets, q, inter, dense_backbone=True)
    osp, ors = sq.grouped_dual_gemm_silu_prepare(sp, rs, wq, torch.from_numpy(offsets).to(DEV), rows,
                                                 row_index=torch.from_numpy(row_index).to(DEV),
                                                 dense_backbone=True)
    _compare_prep("grouped silu residues", osp, ors, ref)


def test_grouped_dual_gemm_bad_offsets_stay_inside_y():
    """Offsets that decrease or run past the row count (possible when routing
    on the device goes wrong) are clamped to [0, rows]: Y's neighbours are
    never written, and rows that only a well-formed group covers are right
    (here group 0 alone owns rows 0-9; group 2's clamped range 10-39 overlaps
    it, so rows 10-29 may hold either group's product)."""
    tokens, k, n = 64, 256, 128
    x = si.activations("normal", tokens, k, 4, 20.0, 81)
    W = si.weights(4 * n, k, 82)
    sp, rs = sq.prepare(dev16(x), None, dense_backbone=True)
    wq = sq.quantize_weight(dev16(W))
    rows = 40
    offsets = torch.tensor([0, 30, 10, 500, 7], dtype=torch.int64, device=DEV)
    buf = torch.full((rows + 64, n), 7.5, dtype=torch.float32, device=DEV)
    out = buf[32:32 + rows]
    sq.grouped_dual_gemm(sp, rs, wq, offsets, rows, out=out)
    got = host(buf)
    assert (got[:32] == 7.5).all() and (got[32 + rows:] == 7.5).all()
    p = oracle.prepare(sq.MXFP4, x, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, W)
    ref, yabs = oracle.grouped_dual_gemm_bound(sq.MXFP4, p, None, [0, 10], q, n)
    check_gemm(got[32:42], ref, yabs, k, "test_grouped_dual_gemm_bad_offsets_stay_inside_y")
    # rows 30-39 belong to group 2 alone: activation rows 30-39 with W rows 2n .. 3n - 1
    ref, yabs = oracle.dual_gemm_bound(sq.MXFP4, oracle.gather_rows(p, np.arange(30, 40)), oracle.expert_rows(q, 2, n))
    check_gemm(got[62:72], ref, yabs, k, "test_grouped_dual_gemm_bad_offsets_stay_inside_y")


def test_grouped_dual_gemm_qwen3_layer_sampled():
    """The bench shape: one Qwen3-30B-A3B MoE layer's gate+up expert GEMMs
    (4096 tokens, 128 experts, 8 a token, n 1536, k 2048), sampled outputs."""
    cfg = si.MOE_QWEN3_30B_A3B
    tokens, k, n, experts = 4096, cfg["hidden"], 2 * cfg["intermediate"], cfg["experts"]
    p, q, sp, rs, wq, row_index, offsets = _grouped_case(tokens, k, n, experts, cfg["top_k"], 91)
    rows = int(offsets[-1])
    y = host(sq.grouped_dual_gemm(sp, rs, wq, torch.from_numpy(offsets).to(DEV), rows,
                                  row_index=torch.from_numpy(row_index).to(DEV)))
    rng = np.random.default_rng(3)
    pick = np.sort(rng.integers(0, rows, 512))
    pick[:2] = [0, rows - 1]
    group_of = np.searchsorted(offsets, pick, side="right") - 1
    got, want, mags = [], [], []
    for e in np.unique(group_of):
        sel = pick[group_of == e]
        cols = rng.integers(0, n, len(sel))
        pe = oracle.gather_rows(p, row_index[sel])
        ref, yabs = oracle.dual_gemm_pairs_bound(sq.MXFP4, pe, oracle.expert_rows(q, int(e), n),
                                                 np.arange(len(sel)), cols)
        got.append(y[sel, cols])
        want.append(ref)
        mags.append(yabs)
    check_gemm(np.concatenate(got), np.concatenate(want), np.concatenate(mags), k,
               "test_grouped_dual_gemm_qwen3_layer_sampled")


# ------------------------------------------------------------ gate+up GEMM with SiLU(gate) * up and the preparation
KSM, ROW = sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR


def _silu_gemm_grid_case(m, inter, k, seed, layout):
    """FP4-grid X [m, k] and W [2 inter, k] (see synth_inputs.fp4_grid): the
    dual GEMM of their FP4 operands is exact in fp32 in any summation order."""
    xb = si.fp4_grid(m, k, 0, seed)
    wb = si.fp4_grid(2 * inter, k, -6, seed + 1)
    sp, rs = sq.prepare(dev16(xb), None, dense_backbone=True, layout=layout)
    wq = sq.quantize_weight(dev16(wb), layout=layout)
    return xb, wb, sp, rs, wq


@pytest.mark.parametrize("m,inter,k,in_layout,out_layout,dense", [
    (200, 256, 384, KSM, KSM, True), (1, 128, 128, KSM, KSM, True), (300, 384, 512, ROW, ROW, True),
    (129, 128, 256, ROW, KSM, False), (256, 512, 1024, KSM, ROW, True), (37, 1024, 256, KSM, KSM, False)])
def test_dual_gemm_silu_prepare_exact(m, inter, k, in_layout, out_layout, dense):
    """The gate+up GEMM with SiLU(gate) * up and the preparation in its
    epilogue, on FP4-grid inputs (the GEMM exact in fp32): every prepared
    array byte for byte against the oracle's GEMM -> SiLU(gate) * up ->
    preparation, in full; ragged m, one to eight column tiles, both layouts
    of the inputs and of the outputs, with and without the dense backbone
    view."""
    xb, wb, sp, rs, wq = _silu_gemm_grid_case(m, inter, k, 71, in_layout)
    p = oracle.prepare(sq.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    _, ref = oracle.dual_gemm_silu_prepare(sq.MXFP4, p, q, dense_backbone=True)
    osp, ors = sq.dual_gemm_silu_prepare(sp, rs, wq, dense_backbone=dense, layout=out_layout)
    _compare_prep(f"silu gemm m{m} inter{inter} k{k}", osp, ors, ref, dense=dense)


def test_dual_gemm_silu_prepare_llama_gate_up_sampled():
    """Llama-3.1-8B's gate+up at prefill (m 2048, inter 14336, k 4096, the
    bench's launch) on FP4-grid inputs: sampled rows of every output array
    byte for byte against the oracle (the preparation is row-independent)."""
    m, inter, k = 2048, 14336, 4096
    xb, wb, sp, rs, wq = _silu_gemm_grid_case(m, inter, k, 81, KSM)
    osp, ors = sq.dual_gemm_silu_prepare(sp, rs, wq, dense_backbone=True)
    rows = np.array([0, 1, 127, 128, 1000, 2047])
    p = oracle.prepare(sq.MXFP4, xb[rows], None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    _, ref = oracle.dual_gemm_silu_prepare(sq.MXFP4, p, q, dense_backbone=True)
    got = {"meta": osp.row_major("meta"), "s_codes": osp.row_major("codes"),
           "s_scales": osp.row_major("scales"), "s_dense": osp.row_major("dense_codes"),
           "r_codes": ors.row_major("codes"), "r_scales": ors.row_major("scales")}
    for key, val in got.items():
        val = host(val)[rows]
        assert np.array_equal(val, ref[key]), (key, int((val != ref[key]).sum()))


def test_dual_gemm_silu_prepare_matches_two_step_path():
    """The layer's own inputs (RMSNorm of heavy-tailed activations with outlier
    channels, N(0, 0.02) weights; fp32 products not exact): the fused entry
    point writes what sharq_dual_gemm followed by sharq_prepare_silu_mul on
    the two halves of Y writes, byte for byte (the same fp32 products, SiLU and
    preparation).  A consistency check between two library paths, each of
    which the tests above hold to the oracle."""
    w = si.layer_workload("gate_up", 2048)
    x, g, W = si.workload_x(w), si.workload_gamma(w), si.workload_w(w)
    inter = W.shape[0] // 2
    sp, rs = sq.prepare(dev16(x), dev16(g), dense_backbone=True)
    wq = sq.quantize_weight(dev16(W))
    osp, ors = sq.dual_gemm_silu_prepare(sp, rs, wq, dense_backbone=True)
    y = sq.dual_gemm(sp, rs, wq)
    tsp, trs = sq.prepare_silu_mul(y[:, :inter], y[:, inter:], dense_backbone=True)
    torch.cuda.synchronize()
    for a, b, name in ((osp.codes, tsp.codes, "s_codes"), (osp.meta, tsp.meta, "meta"),
                       (osp.scales, tsp.scales, "s_scales"), (osp.dense_codes, tsp.dense_codes, "s_dense"),
                       (ors.codes, trs.codes, "r_codes"), (ors.scales, trs.scales, "r_scales")):
        assert torch.equal(a, b), (name, int((a != b).sum()))


def _grouped_silu_grid_case(tokens, k, inter, experts, top_k, seed, layout):
    xb = si.fp4_grid(tokens, k, 0, seed)
    wb = si.fp4_grid(experts * 2 * inter, k, -6, seed + 1)
    row_index, offsets = si.moe_routing(tokens, experts, top_k, seed + 2)
    sp, rs = sq.prepare(dev16(xb), None, dense_backbone=True, layout=layout)
    wq = sq.quantize_weight(dev16(wb), layout=layout)
    return xb, wb, row_index, offsets, sp, rs, wq


@pytest.mark.parametrize("tokens,k,inter,experts,top_k,layout", [
    (300, 256, 128, 8, 2, KSM), (200, 384, 256, 5, 3, ROW), (64, 128, 384, 16, 4, KSM)])
def test_grouped_dual_gemm_silu_prepare_exact(tokens, k, inter, experts, top_k, layout):
    """The grouped gate+up GEMMs with SiLU(gate) * up and the preparation in
    the epilogue, on FP4-grid inputs (every product exact in fp32): every
    prepared array of every grouped row byte for byte against the oracle's
    grouped GEMM -> SiLU(gate) * up -> preparation; seeded routing with uneven
    groups, both layouts."""
    xb, wb, row_index, offsets, sp, rs, wq = _grouped_silu_grid_case(tokens, k, inter, experts, top_k, 101, layout)
    rows = int(offsets[-1])
    p = oracle.prepare(sq.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    _, ref = oracle.grouped_dual_gemm_silu_prepare(sq.MXFP4, p, row_index, offsets, q, inter, dense_backbone=True)
    osp, ors = sq.grouped_dual_gemm_silu_prepare(sp, rs, wq, torch.from_numpy(offsets).to(DEV), rows,
                                                 row_index=torch.from_numpy(row_index).to(DEV),
                                                 dense_backbone=True, layout=layout)
    _compare_prep(f"grouped silu t{tokens} k{k} inter{inter}", osp, ors, ref)


def test_grouped_dual_gemm_silu_prepare_identity_and_empty_groups():
    """Identity gather (no row index) with empty groups at the start, middle
    and end: the same bytes as the oracle."""
    tokens, k, inter = 150, 256, 128
    xb, wb, _, _, sp, rs, wq = _grouped_silu_grid_case(tokens, k, inter, 5, 1, 111, KSM)
    offsets = np.array([0, 0, 70, 70, 150, 150], dtype=np.int64)
    p = oracle.prepare(sq.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    _, ref = oracle.grouped_dual_gemm_silu_prepare(sq.MXFP4, p, None, offsets, q, inter, dense_backbone=True)
    osp, ors = sq.grouped_dual_gemm_silu_prepare(sp, rs, wq, torch.from_numpy(offsets).to(DEV), tokens,
                                                 dense_backbone=True)
    _compare_prep("grouped silu identity", osp, ors, ref)


def test_grouped_dual_gemm_silu_prepare_qwen3_layer():
    """The MoE bench shape (4096 tokens, 128 experts, 8 a token, inter 768, k
    2048): on FP4-grid inputs, sampled grouped rows byte for byte against the
    oracle; on the layer's own inputs, every byte equal to the grouped GEMM
    followed by sharq_prepare_silu_mul (a consistency check between two
    library paths)."""
    cfg = si.MOE_QWEN3_30B_A3B
    tokens, k, inter, experts, top_k = 4096, cfg["hidden"], cfg["intermediate"], cfg["experts"], cfg["top_k"]
    xb, wb, row_index, offsets, sp, rs, wq = _grouped_silu_grid_case(tokens, k, inter, experts, top_k, 121, KSM)
    rows = int(offsets[-1])
    doff, didx = torch.from_numpy(offsets).to(DEV), torch.from_numpy(row_index).to(DEV)
    osp, ors = sq.grouped_dual_gemm_silu_prepare(sp, rs, wq, doff, rows, row_index=didx, dense_backbone=True)
    got = {"meta": host(osp.row_major("meta")), "s_codes": host(osp.row_major("codes")),
           "s_scales": host(osp.row_major("scales")), "s_dense": host(osp.row_major("dense_codes")),
           "r_codes": host(ors.row_major("codes")), "r_scales": host(ors.row_major("scales"))}
    rng = np.random.default_rng(7)
    pick = np.concatenate([[0, rows - 1], rng.integers(0, rows, 22)])
    for i in pick:
        e = int(np.searchsorted(offsets, i, side="right") - 1)
        # the preparation and the weight quantization are row-independent:
        # the oracle prepares the one token and quantizes the one expert
        p = oracle.prepare(sq.MXFP4, xb[row_index[i]:row_index[i] + 1], None, dense_backbone=True)
        q = oracle.quantize_weight(sq.MXFP4, wb[e * 2 * inter:(e + 1) * 2 * inter])
        _, ref = oracle.dual_gemm_silu_prepare(sq.MXFP4, p, q, dense_backbone=True)
        for key, val in got.items():
            assert np.array_equal(val[i], ref[key][0]), (int(i), e, key)
    # the layer's own inputs: fused against the two library steps
    x = si.activations("student_t4", tokens, k, 41, 50.0, 131)
    g = si.gamma(k, 132)
    W = si.weights(experts * 2 * inter, k, 133)
    sp, rs = sq.prepare(dev16(x), dev16(g), dense_backbone=True)
    wq = sq.quantize_weight(dev16(W))
    osp, ors = sq.grouped_dual_gemm_silu_prepare(sp, rs, wq, doff, rows, row_index=didx, dense_backbone=True)
    y = sq.grouped_dual_gemm(sp, rs, wq, doff, rows, row_index=didx)
    tsp, trs = sq.prepare_silu_mul(y[:, :inter], y[:, inter:], dense_backbone=True)
    torch.cuda.synchronize()
    for a, b, name in ((osp.codes, tsp.codes, "s_codes"), (osp.meta, tsp.meta, "meta"),
                       (osp.scales, tsp.scales, "s_scales"), (osp.dense_codes, tsp.dense_codes, "s_dense"),
                       (ors.codes, trs.codes, "r_codes"), (ors.scales, trs.scales, "r_scales")):
        assert torch.equal(a, b), (name, int((a != b).sum()))


# ------------------------------------------------------------ weights
@pytest.mark.parametrize("fmt,n,k", [(0, 256, 256), (0, 6144, 4096), (0, 33, 96), (1, 256, 256),
                                     (1, 1000, 4096)])
def test_quantize_weight(fmt, n, k):
    w = si.weights(n, k, seed=n + k)
    ref = oracle.quantize_weight(fmt, w)
    layouts = [sq.LAYOUT_ROW_MAJOR] + ([sq.LAYOUT_KSTEP_MAJOR] if k % 128 == 0 else [])
    for layout in layouts:
        got = sq.quantize_weight(dev16(w), fmt, layout=layout)
        assert np.array_equal(host(got.row_major("codes")), ref["codes"])
        assert np.array_equal(host(got.row_major("scales")), ref["scales"])
    if fmt == sq.NVFP4:
        assert host(got.tensor_scale)[0] == ref["tensor_scale"][0]


# ------------------------------------------------------------ GEMM
# MXFP4: the backbone's dense view, the 2:4 form expanded in LDS, and the 2:4
# form rebased to FP8 on the structured-sparse FP8 MFMA
MX_VARIANTS = (sq.GEMM_DECOMPRESS, sq.GEMM_DENSE_EXPANDED, sq.GEMM_SPARSE_MFMA)


def _gemm_case(m, n, k, seed, fmt=sq.MXFP4, norm=True):
    x = si.activations("student_t4", m, k, max(1, k // 100), 50.0, seed=seed)
    w = si.weights(n, k, seed=seed + 1)
    g = si.gamma(k, seed + 2) if norm else None
    p = oracle.prepare(fmt, x, g, dense_backbone=True)
    q = oracle.quantize_weight(fmt, w)
    return x, w, g, p, q


@pytest.mark.parametrize("m,n,k", [(16, 256, 256), (37, 75, 256), (130, 200, 384), (1, 1, 128),
                                   (257, 129, 1024), (64, 512, 4096), (300, 1000, 640),
                                   (129, 193, 128), (512, 192, 256), (32, 300, 640), (7, 96, 1152),
                                   (33, 64, 384)])
def test_dual_gemm_mx_vs_oracle(m, n, k):
    x, w, g, p, q = _gemm_case(m, n, k, seed=m + 7 * n + k)
    ref, yabs = oracle.dual_gemm_bound(sq.MXFP4, p, q)
    for layout in (sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR):
        sp, rs = to_dev_prep(sq.MXFP4, p, layout)
        wq = to_dev_weight(sq.MXFP4, q, layout)
        for variant in MX_VARIANTS:
            y = host(sq.dual_gemm(sp, rs, wq, variant=variant))
            check_gemm(y, ref, yabs, k, f"test_dual_gemm_mx_vs_oracle {layout} {variant}")


@pytest.mark.parametrize("m,n,k", [(2000, 6100, 384), (2000, 4000, 640), (2048, 4096, 128)])
def test_dual_gemm_mx_large_tile_configs(m, n, k):
    """Shapes that take the tile configurations of the large workloads
    (128 x 192 for both variants; 128 x 128 dense and 128 x 256 expanding),
    with ragged edges, against the oracle at every 32-row and 32-column tile
    edge plus random outputs."""
    x, w, g, p, q = _gemm_case(m, n, k, seed=m + n + k)
    rng = np.random.default_rng(m + n)
    er = np.concatenate([np.arange(0, m, 32), np.arange(31, m, 32), [m - 1]])
    ec = np.concatenate([np.arange(0, n, 32), np.arange(31, n, 32), [n - 1]])
    rows = np.concatenate([er, rng.integers(0, m, 4000), rng.integers(0, m, ec.size)])
    cols = np.concatenate([rng.integers(0, n, er.size), rng.integers(0, n, 4000), ec])
    order = np.argsort(rows, kind="stable")
    rows, cols = rows[order], cols[order]
    ref, yabs = oracle.dual_gemm_pairs_bound(sq.MXFP4, p, q, rows, cols)
    for layout in (sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR):
        sp, rs = to_dev_prep(sq.MXFP4, p, layout)
        wq = to_dev_weight(sq.MXFP4, q, layout)
        ys = [host(sq.dual_gemm(sp, rs, wq, variant=v)) for v in MX_VARIANTS]
        for v, y in zip(("decompress", "dense", "sparse_fp8"), ys):
            assert np.isfinite(y).all(), (layout, v)
            check_gemm(y[rows, cols], ref, yabs, k, f"test_dual_gemm_mx_large_tile_configs {layout} {v}")


@pytest.mark.parametrize("m,n,k", [(16, 16384 + 64 + 5, 256), (17, 16384 + 64 + 5, 384), (32, 20000, 128),
                                   (1, 16448, 256), (9, 32768 + 128 + 3, 256), (32, 32768 + 128, 128)])
def test_dual_gemm_decode_kernel(m, n, k):
    """The decode kernel (m <= 32, dense view, at least 128 column tiles of
    128): one A chunk (m <= 16) or two, ragged last tiles, both layouts.
    Every output."""
    x, w, g, p, q = _gemm_case(m, n, k, seed=m + n + k)
    ref, yabs = oracle.dual_gemm_bound(sq.MXFP4, p, q)
    for layout in (sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR):
        sp, rs = to_dev_prep(sq.MXFP4, p, layout)
        wq = to_dev_weight(sq.MXFP4, q, layout)
        y = host(sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_DENSE_EXPANDED))
        check_gemm(y, ref, yabs, k, f"test_dual_gemm_decode_kernel {layout}")


def test_dual_gemm_variants_bitwise_equal():
    x, w, g, p, q = _gemm_case(200, 300, 512, seed=3)
    sp, rs = to_dev_prep(sq.MXFP4, p, sq.LAYOUT_ROW_MAJOR)
    wq = to_dev_weight(sq.MXFP4, q, sq.LAYOUT_ROW_MAJOR)
    a = sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_DECOMPRESS)
    b = sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_DENSE_EXPANDED)
    c = sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_DECOMPRESS)
    assert torch.equal(a, b) and torch.equal(a, c)
    # the k-step-major pipeline: deterministic run to run
    sp2, rs2 = to_dev_prep(sq.MXFP4, p, sq.LAYOUT_KSTEP_MAJOR)
    wq2 = to_dev_weight(sq.MXFP4, q, sq.LAYOUT_KSTEP_MAJOR)
    d = sq.dual_gemm(sp2, rs2, wq2, variant=sq.GEMM_DENSE_EXPANDED)
    e = sq.dual_gemm(sp2, rs2, wq2, variant=sq.GEMM_DENSE_EXPANDED)
    assert torch.equal(d, e)


def test_dual_gemm_exact_special_case():
    """2:4-sparse FP4-representable X and FP4 W: the product is exact in fp32,
    so the GPU must match the oracle bit for bit."""
    rng = np.random.default_rng(5)
    m, k, n = 64, 256, 96
    from brute import e2m1_value
    xv = e2m1_value(rng.integers(0, 16, (m, k)))
    for i in range(m):
        for gi in range(k // 4):
            xv[i, 4 * gi + rng.choice(4, 2, replace=False)] = 0.0
    xv = np.where(xv == 0, 0.0, xv) * 2.0 ** rng.integers(-3, 3, (m, 1))
    wv = e2m1_value(rng.integers(0, 16, (n, k))) * 2.0 ** rng.integers(-8, -4, (n, 1))
    xb = si.f32_to_bf16_bits(xv.astype(np.float32))
    wb = si.f32_to_bf16_bits(wv.astype(np.float32))
    p = oracle.prepare(sq.MXFP4, xb, None)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    ref, yabs = oracle.dual_gemm_bound(sq.MXFP4, p, q)
    assert (ref == (xv @ wv.T).astype(np.float32)).all()
    sp, rs = sq.prepare(dev16(xb), None, dense_backbone=True)
    wq = sq.quantize_weight(dev16(wb))
    for variant in (sq.GEMM_AUTO, *MX_VARIANTS):
        y = host(sq.dual_gemm(sp, rs, wq, variant=variant))
        assert np.array_equal(y, ref), variant
        check_gemm(y, ref, yabs, k, "test_dual_gemm_exact_special_case")


def _check_end_to_end(w, samples):
    """prepare + dual GEMM (dense view and DECOMPRESS) on the GPU vs the
    oracle's, at the workload's full size (sampled outputs when `samples`)."""
    x, W, g = si.workload_x(w), si.workload_w(w), si.workload_gamma(w)
    p = oracle.prepare(sq.MXFP4, x, g)
    q = oracle.quantize_weight(sq.MXFP4, W)
    sp, rs = sq.prepare(dev16(x), None if g is None else dev16(g), dense_backbone=True)
    wq = sq.quantize_weight(dev16(W))
    y = host(sq.dual_gemm(sp, rs, wq))
    y2 = host(sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_DECOMPRESS))
    y3 = host(sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_SPARSE_MFMA))
    if samples is None:
        ref, yabs = oracle.dual_gemm_bound(sq.MXFP4, p, q)
        check_gemm(y2, ref, yabs, w.k, "end_to_end decompress")
        check_gemm(y, ref, yabs, w.k, "end_to_end dense")
        check_gemm(y3, ref, yabs, w.k, "end_to_end sparse_fp8")
        return
    rng = np.random.default_rng(0)
    rows = np.sort(rng.integers(0, w.m, samples))
    cols = rng.integers(0, w.n, samples)
    rows[:4] = [0, 0, w.m - 1, w.m - 1]
    cols[:4] = [0, w.n - 1, 0, w.n - 1]
    order = np.argsort(rows, kind="stable")
    rows, cols = rows[order], cols[order]
    ref, yabs = oracle.dual_gemm_pairs_bound(sq.MXFP4, p, q, rows, cols)
    # normwise: normalized by the largest |Y| over the sample (the full max is at least this)
    check_gemm(y[rows, cols], ref, yabs, w.k, "end_to_end dense")
    check_gemm(y2[rows, cols], ref, yabs, w.k, "end_to_end decompress")
    check_gemm(y3[rows, cols], ref, yabs, w.k, "end_to_end sparse_fp8")


@pytest.mark.parametrize("name,samples", [("tiny", None), ("qkv_prefill", 4096),
                                          ("down_prefill", 4096), ("decode_gate_up", 8192)])
def test_end_to_end_workloads(name, samples):
    _check_end_to_end(si.WORKLOADS[name], samples)


@pytest.mark.parametrize("linear,m,samples", [("o", 2048, 4096), ("gate_up", 2048, 4096),
                                              ("qkv", 16, None), ("o", 16, None), ("down", 16, None)])
def test_layer_chain_linears(linear, m, samples):
    """The decoder-layer chain's other shapes (bench.py --chain): O projection
    (no norm, plain normal input), gate+up at prefill, and the decode shapes."""
    _check_end_to_end(si.layer_workload(linear, m), samples)


def _padded(t, layout, extra_rows=0, extra_bytes=0):
    """A copy of device array `t` inside a larger buffer: row-major arrays get
    `extra_bytes` of padding per row, k-step-major ones `extra_rows` rows per step."""
    if layout == sq.LAYOUT_KSTEP_MAJOR:
        steps, rows, bps = t.shape
        big = torch.full((steps, rows + extra_rows, bps), 0xA5, dtype=torch.uint8, device=DEV)
        big[:, :rows] = t
        return big[:, :rows]
    rows, nb = t.shape
    big = torch.full((rows, nb + extra_bytes), 0xA5, dtype=torch.uint8, device=DEV)
    big[:, :nb] = t
    return big[:, :nb]


@pytest.mark.parametrize("fmt", [sq.MXFP4, sq.NVFP4])
@pytest.mark.parametrize("m,n,k", [(96, 160, 384), (20, 200, 256)])
def test_dual_gemm_padded_leading_dims(fmt, m, n, k):
    """Operands inside larger buffers (padding filled with 0xA5): row-major
    rows longer than the data, k-step-major steps with more rows than the
    operand; the GEMM must read only the described bytes."""
    x, w, g, p, q = _gemm_case(m, n, k, seed=m + n, fmt=fmt)
    ref, yabs = oracle.dual_gemm_bound(fmt, p, q)
    variants = NV_VARIANTS if fmt == sq.NVFP4 else MX_VARIANTS
    for layout in (sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR):
        sp, rs = to_dev_prep(fmt, p, layout)
        wq = to_dev_weight(fmt, q, layout)
        pad = dict(extra_rows=24, extra_bytes=48)
        for t in (sp, rs, wq):
            t.codes = _padded(t.codes, layout, **pad)
            t.scales = _padded(t.scales, layout, **pad)
        sp.meta = _padded(sp.meta, layout, **pad)
        sp.dense_codes = _padded(sp.dense_codes, layout, **pad)
        out = torch.full((m, n + 8), float("nan"), dtype=torch.float32, device=DEV)
        for variant in variants:
            y = host(sq.dual_gemm(sp, rs, wq, variant=variant, out=out[:, :n]))
            check_gemm(y[:, :n], ref, yabs, k, f"test_dual_gemm_padded_leading_dims {layout} {variant}")
        assert np.isnan(host(out)[:, n:]).all()        # nothing written past n


@pytest.mark.parametrize("layout", [sq.LAYOUT_ROW_MAJOR, sq.LAYOUT_KSTEP_MAJOR])
def test_dual_gemm_silu_prepare_padded_leading_dims(layout):
    """The fused gate+up entry point with every input and output array inside
    a larger buffer (padding 0xA5): outputs byte for byte equal to the
    oracle's on FP4-grid inputs, and the padding untouched."""
    m, inter, k = 140, 256, 384
    xb, wb, sp, rs, wq = _silu_gemm_grid_case(m, inter, k, 151, layout)
    p = oracle.prepare(sq.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    _, ref = oracle.dual_gemm_silu_prepare(sq.MXFP4, p, q, dense_backbone=True)
    pad = dict(extra_rows=24, extra_bytes=48)
    for t in (sp, rs, wq):
        t.codes = _padded(t.codes, layout, **pad)
        t.scales = _padded(t.scales, layout, **pad)
    sp.meta = _padded(sp.meta, layout, **pad)
    sp.dense_codes = _padded(sp.dense_codes, layout, **pad)
    osp, ors = sq.alloc_prepared(sq.MXFP4, m, inter, DEV, dense_backbone=True, layout=layout)
    for t in (osp, ors):
        t.codes = _padded(t.codes, layout, **pad)
        t.scales = _padded(t.scales, layout, **pad)
    osp.meta = _padded(osp.meta, layout, **pad)
    osp.dense_codes = _padded(osp.dense_codes, layout, **pad)
    sq.bind_dual_gemm_silu_prepare(sp, rs, wq, osp, ors)()
    _compare_prep(f"silu gemm padded {layout}", osp, ors, ref)
    for t in (osp.codes, osp.meta, osp.scales, osp.dense_codes, ors.codes, ors.scales):
        base = t._base                     # the padded buffer: dim 1 is rows (k-step-major) or bytes
        pad_mask = torch.ones_like(base, dtype=torch.bool)
        pad_mask[:, :t.shape[1]] = False
        assert bool((base[pad_mask] == 0xA5).all()), layout


NV_VARIANTS = (sq.GEMM_DECOMPRESS, sq.GEMM_DENSE_EXPANDED, sq.GEMM_SPARSE_MFMA)


@pytest.mark.parametrize("m,n,k", [(16, 256, 256), (37, 75, 256), (1, 1, 128), (130, 200, 384),
                                   (257, 129, 1024), (64, 512, 4096), (300, 1000, 640),
                                   (129, 193, 128), (512, 768, 256)])
def test_dual_gemm_nv_vs_oracle(m, n, k):
    """NVFP4-style dual GEMM, all three backbone variants, both scale layouts."""
    x, w, g, p, q = _gemm_case(m, n, k, seed=3 * m + n + k, fmt=sq.NVFP4)
    ref, yabs = oracle.dual_gemm_bound(sq.NVFP4, p, q)
    for layout in (sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR):
        sp, rs = to_dev_prep(sq.NVFP4, p, layout)
        wq = to_dev_weight(sq.NVFP4, q, layout)
        for variant in NV_VARIANTS:
            y = host(sq.dual_gemm(sp, rs, wq, variant=variant))
            check_gemm(y, ref, yabs, k, f"test_dual_gemm_nv_vs_oracle {layout} {variant}")


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 300)), int(rng.integers(1, 400)), 128 * int(rng.integers(1, 5)))
            for _ in range(count)]


@pytest.mark.parametrize("fmt", [sq.MXFP4, sq.NVFP4])
def test_dual_gemm_random_shapes(fmt):
    """Seeded random shapes (m 1-299, n 1-399, k 128-512, both layouts, every
    variant): ragged tiles in every position, the decode / prefill switch at
    m = 32 and single-step K."""
    variants = NV_VARIANTS if fmt == sq.NVFP4 else MX_VARIANTS
    for i, (m, n, k) in enumerate(_random_shapes(11 + fmt, 10)):
        x, w, g, p, q = _gemm_case(m, n, k, seed=1000 + i, fmt=fmt, norm=bool(i % 2))
        ref, yabs = oracle.dual_gemm_bound(fmt, p, q)
        layout = (sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR)[i % 2]
        sp, rs = to_dev_prep(fmt, p, layout)
        wq = to_dev_weight(fmt, q, layout)
        for variant in variants:
            y = host(sq.dual_gemm(sp, rs, wq, variant=variant))
            check_gemm(y, ref, yabs, k, f"test_dual_gemm_random_shapes {m} {n} {k} {layout} {variant}")


def test_dual_gemm_nv_dense_and_expanded_bitwise_equal():
    """The expanded 2:4 backbone and the dense view feed identical MFMAs."""
    x, w, g, p, q = _gemm_case(200, 600, 512, seed=11, fmt=sq.NVFP4)
    sp, rs = to_dev_prep(sq.NVFP4, p)
    wq = to_dev_weight(sq.NVFP4, q)
    a = sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_DECOMPRESS)
    b = sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_DENSE_EXPANDED)
    c = sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_SPARSE_MFMA)
    d = sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_SPARSE_MFMA)
    assert torch.equal(a, b)
    assert torch.equal(c, d)


def _zeroed(p, which):
    """Copy of oracle preparation outputs with one path's codes set to 0 (+0.0)."""
    z = dict(p)
    if which == "backbone":
        z["s_codes"] = np.zeros_like(p["s_codes"])
        if "s_dense" in p:
            z["s_dense"] = np.zeros_like(p["s_dense"])
    else:
        z["r_codes"] = np.zeros_like(p["r_codes"])
    return z


@pytest.mark.parametrize("fmt", [sq.MXFP4, sq.NVFP4])
def test_dual_gemm_path_specific_weight_views(fmt):
    """Distinct scale views of one W payload: the backbone product reads the
    sparse-path view, the residual product the dense-path view."""
    m, n, k = 96, 320, 512
    x, w, g, p, q = _gemm_case(m, n, k, seed=21, fmt=fmt)
    q2 = dict(q)
    rng = np.random.default_rng(4)
    if fmt == sq.MXFP4:
        q2["scales"] = (q["scales"].astype(np.int32) + rng.integers(-2, 3, q["scales"].shape)).clip(1, 254).astype(np.uint8)
    else:   # positive finite E4M3 bytes
        q2["scales"] = rng.integers(0x08, 0x70, q["scales"].shape).astype(np.uint8)
    ya, abs_a = oracle.dual_gemm_bound(fmt, _zeroed(p, "residual"), q)
    yb, abs_b = oracle.dual_gemm_bound(fmt, _zeroed(p, "backbone"), q2)
    ref, yabs = ya.astype(np.float64) + yb, abs_a + abs_b
    variants = NV_VARIANTS if fmt == sq.NVFP4 else MX_VARIANTS
    for layout in (sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR):
        sp, rs = to_dev_prep(fmt, p, layout)
        wq = to_dev_weight(fmt, q, layout)
        wd = dev_scales(q2["scales"], fmt, layout)
        for variant in variants:
            y = host(sq.dual_gemm(sp, rs, wq, variant=variant, w_dense_scales=wd))
            check_gemm(y, ref, yabs, k, f"test_dual_gemm_path_specific_weight_views {layout} {variant}")


@pytest.mark.parametrize("name,samples", [("tiny", None), ("nvfp4_prefill", 4096)])
def test_end_to_end_nv_workloads(name, samples):
    """NVFP4-style prepare + weight quantization + dual GEMM on the GPU vs the
    oracle's, every variant."""
    w = si.WORKLOADS[name]
    x, W, g = si.workload_x(w), si.workload_w(w), si.workload_gamma(w)
    p = oracle.prepare(sq.NVFP4, x, g)
    q = oracle.quantize_weight(sq.NVFP4, W)
    sp, rs = sq.prepare(dev16(x), None if g is None else dev16(g), fmt=sq.NVFP4, dense_backbone=True)
    wq = sq.quantize_weight(dev16(W), fmt=sq.NVFP4)
    ys = [host(sq.dual_gemm(sp, rs, wq, variant=v)) for v in NV_VARIANTS]
    if samples is None:
        ref, yabs = oracle.dual_gemm_bound(sq.NVFP4, p, q)
        for v, y in zip(NV_VARIANTS, ys):
            check_gemm(y, ref, yabs, w.k, f"test_end_to_end_nv_workloads {v}")
        return
    rng = np.random.default_rng(1)
    rows = np.sort(rng.integers(0, w.m, samples))
    cols = rng.integers(0, w.n, samples)
    rows[:4] = [0, 0, w.m - 1, w.m - 1]
    cols[:4] = [0, w.n - 1, 0, w.n - 1]
    order = np.argsort(rows, kind="stable")
    rows, cols = rows[order], cols[order]
    ref, yabs = oracle.dual_gemm_pairs_bound(sq.NVFP4, p, q, rows, cols)
    for v, y in zip(NV_VARIANTS, ys):
        check_gemm(y[rows, cols], ref, yabs, w.k, f"test_end_to_end_nv_workloads {v}")


def _blocks_at(v, exps):
    """v [rows, k] with each 32-block rescaled so that its largest magnitude is
    5 * 2^e (e from exps [rows, k / 32]): its MX scale exponent is then e."""
    rows, k = v.shape
    b = v.reshape(rows, k // 32, 32).astype(np.float64)
    b = b / np.abs(b).max(axis=2, keepdims=True) * 5.0 * 2.0 ** exps[..., None]
    return b.reshape(rows, k).astype(np.float32)


@pytest.mark.parametrize("layout", [sq.LAYOUT_KSTEP_MAJOR, sq.LAYOUT_ROW_MAJOR])
def test_dual_gemm_mx_sparse_fp8_rebasing_and_fallback(layout):
    """SPARSE_MFMA for MXFP4: tiles whose A rows and W rows each span at most
    12 block exponents run the backbone rebased to FP8 on the 2:4 FP8 MFMA
    (here spans of exactly 12, so the lowest blocks sit 7 below the reference
    and their FP8 values are subnormal); a tile with an A row or a W row
    spanning more falls back to the expanded FP4 backbone.  Tiles of 128:
    A row 5 spans 16 (tile row 0 falls back), rows 128-299 span 12; W row 200
    spans 22 (tile column 1 falls back), the other rows 12."""
    m, n, k = 300, 400, 512
    rng = np.random.default_rng(12)
    ex = np.zeros((m, k // 32), np.int64)
    ex[128:, 3], ex[128:, 9] = 6, -6
    ex[5, 2] = 16
    x = _blocks_at(rng.standard_normal((m, k)), ex)
    ew = np.full((n, k // 32), -6, np.int64)
    ew[:, 1], ew[:, 14] = 0, -12
    ew[200, 7] = 10
    w = _blocks_at(rng.standard_normal((n, k)), ew)
    xb, wb = si.f32_to_bf16_bits(x), si.f32_to_bf16_bits(w)
    p = oracle.prepare(sq.MXFP4, xb, None, dense_backbone=True)
    q = oracle.quantize_weight(sq.MXFP4, wb)
    span = lambda sc: sc.max(axis=1).astype(int) - sc.min(axis=1).astype(int)
    assert span(p["s_scales"])[5] == 16 and (span(p["s_scales"])[128:] == 12).all()
    assert span(q["scales"])[200] == 22 and (span(q["scales"])[np.arange(n) != 200] == 12).all()
    ref, yabs = oracle.dual_gemm_bound(sq.MXFP4, p, q)
    sp, rs = to_dev_prep(sq.MXFP4, p, layout)
    wq = to_dev_weight(sq.MXFP4, q, layout)
    y = host(sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_SPARSE_MFMA))
    check_gemm(y, ref, yabs, k, f"test_dual_gemm_mx_sparse_fp8 {layout}")
    # repeatable bit for bit
    assert np.array_equal(host(sq.dual_gemm(sp, rs, wq, variant=sq.GEMM_SPARSE_MFMA)), y)
