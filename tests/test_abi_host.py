"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid requests before any HIP call (every
request here fails validation, so nothing reaches the GPU)."""
import ctypes
import os
import re

import pytest

import sparsity_fp4_quantized_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "sharq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sharq_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    L = sq.lib()
    names = header_functions()
    assert set(names) == set(sq.EXPORTS), names
    for name in names:
        assert hasattr(L, name), name
    assert L.sharq_abi_version() == sq.ABI_VERSION


def test_yardstick_library_loads():
    """bench.py's measurement library (not part of the ABI) is built beside the
    product library and exports its one entry point."""
    path = os.path.join(os.path.dirname(sq.LIB_PATH), "libsharq_yardstick.so")
    L = ctypes.CDLL(path)
    assert hasattr(L, "sharq_yardstick_mfma_fp4")
    # invalid arguments are refused before any launch
    L.sharq_yardstick_mfma_fp4.restype = ctypes.c_int
    assert L.sharq_yardstick_mfma_fp4(0, 1, 1, None, None, None) != 0
    assert hasattr(L, "sharq_yardstick_stream_read")
    L.sharq_yardstick_stream_read.restype = ctypes.c_int
    L.sharq_yardstick_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert L.sharq_yardstick_stream_read(None, 16384, None, None) != 0
    assert L.sharq_yardstick_stream_read(1 << 20, 1000, 1 << 20, None) != 0


def test_status_strings_and_sizes():
    for s in range(6):
        assert sq.status_str(s)
    assert sq.status_str(99) == "unknown status"
    assert sq.nbytes(sq.MXFP4, sq.BYTES_DENSE_CODES, 16, 256) == 16 * 128
    assert sq.nbytes(sq.MXFP4, sq.BYTES_SPARSE_CODES, 16, 256) == 16 * 64
    assert sq.nbytes(sq.MXFP4, sq.BYTES_META, 16, 256) == 16 * 32
    assert sq.nbytes(sq.MXFP4, sq.BYTES_SCALES, 16, 256) == 16 * 8
    assert sq.nbytes(sq.NVFP4, sq.BYTES_SCALES, 16, 256) == 16 * 16
    assert sq.nbytes(sq.MXFP4, 9, 16, 256) == 0
    assert sq.nbytes(sq.MXFP4, 0, 16, 100) == 0


FAKE = 1 << 20     # aligned, never dereferenced: validation fails first


def view(codes=FAKE, ld_codes=128, meta=FAKE, ld_meta=32, scales=FAKE, ld_scales=8,
         dense=None, ld_dense=0, ts=None, layout=0, reserved=0):
    v = sq.FP4ViewC()
    v.codes, v.ld_codes, v.meta, v.ld_meta = codes, ld_codes, meta, ld_meta
    v.scales, v.ld_scales, v.dense_codes, v.ld_dense, v.tensor_scale = scales, ld_scales, dense, ld_dense, ts
    v.layout, v.reserved = layout, reserved
    return v


def ksm(rows=16, **kw):
    """A k-step-major view: every ld counts rows per 128-k step."""
    args = dict(ld_codes=rows, ld_meta=rows, ld_scales=rows, layout=sq.LAYOUT_KSTEP_MAJOR)
    args.update(kw)
    return view(**args)


def prep(fmt=0, x=FAKE, m=16, k=256, ld_x=256, gamma=None, sp=None, rs=None):
    sp = sp or view(ld_codes=64)
    rs = rs or view(meta=None)
    return sq.lib().sharq_prepare(fmt, x, m, k, ld_x, gamma, 1e-5, ctypes.byref(sp),
                                  ctypes.byref(rs), None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), sq.ERR_NULL),
    (dict(m=0), sq.ERR_SHAPE),
    (dict(k=100, ld_x=100), sq.ERR_SHAPE),
    (dict(k=0), sq.ERR_SHAPE),
    (dict(ld_x=128), sq.ERR_SHAPE),
    (dict(ld_x=260), sq.ERR_ALIGN),
    (dict(x=FAKE + 2), sq.ERR_ALIGN),
    (dict(k=32768, ld_x=32768, gamma=FAKE), sq.ERR_UNSUPPORTED),
    (dict(ld_x=1 << 26), sq.ERR_UNSUPPORTED),   # row strides below 2^26 (32-bit lane offsets)
    (dict(fmt=7), sq.ERR_UNSUPPORTED),
    (dict(sp=view(ld_codes=63)), sq.ERR_SHAPE),
    (dict(sp=view(ld_codes=64, meta=None)), sq.ERR_NULL),
    (dict(sp=view(ld_codes=64, meta=FAKE + 1)), sq.ERR_ALIGN),
    (dict(rs=view(meta=None, codes=FAKE + 8)), sq.ERR_ALIGN),
    (dict(rs=view(meta=None, scales=None)), sq.ERR_NULL),
    (dict(fmt=1), sq.ERR_SHAPE),           # NVFP4 needs k/16 scales per row
    (dict(fmt=1, sp=view(ld_codes=64, ld_scales=16), rs=view(meta=None, ld_scales=16)),
     sq.ERR_NULL),                         # NVFP4 without a tensor-scale buffer
    (dict(sp=ksm(), rs=view(meta=None)), sq.ERR_SHAPE),    # the two views differ in layout
    (dict(k=160, ld_x=160, sp=ksm(), rs=ksm(meta=None)), sq.ERR_SHAPE),   # k % 128
    (dict(sp=ksm(ld_codes=8), rs=ksm(meta=None)), sq.ERR_SHAPE),          # ld < rows
    (dict(sp=ksm(meta=FAKE + 8), rs=ksm(meta=None)), sq.ERR_ALIGN),
    (dict(sp=view(ld_codes=64, reserved=1)), sq.ERR_SHAPE),
    (dict(sp=view(ld_codes=64, layout=5)), sq.ERR_UNSUPPORTED),
])
def test_prepare_validation(kwargs, status):
    assert prep(**kwargs) == status
    assert prep(**kwargs) == status


def prep_res(fmt=0, h=FAKE, ld_h=256, o=FAKE, ld_o=256, out=FAKE, ld_out=256, m=16, k=256,
             gamma=FAKE, sp=None, rs=None):
    sp = sp or view(ld_codes=64)
    rs = rs or view(meta=None)
    return sq.lib().sharq_prepare_residual(fmt, h, ld_h, o, ld_o, out, ld_out, m, k, gamma, 1e-5,
                                           ctypes.byref(sp), ctypes.byref(rs), None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(fmt=1), sq.ERR_UNSUPPORTED),     # NVFP4: the tensor-scale pre-pass would need the sum
    (dict(fmt=7), sq.ERR_UNSUPPORTED),
    (dict(gamma=None), sq.ERR_NULL),       # the norm is part of the fused step
    (dict(h=None), sq.ERR_NULL),
    (dict(o=None), sq.ERR_NULL),
    (dict(out=None), sq.ERR_NULL),
    (dict(ld_o=128), sq.ERR_SHAPE),
    (dict(ld_out=128), sq.ERR_SHAPE),
    (dict(ld_o=260), sq.ERR_ALIGN),
    (dict(o=FAKE + 2), sq.ERR_ALIGN),
    (dict(out=FAKE + 8), sq.ERR_ALIGN),
    (dict(ld_out=264), sq.ERR_SHAPE),      # in place on h (out == h) with another row stride
    (dict(o=FAKE + 4096, ld_out=264, out=FAKE + 4096), sq.ERR_SHAPE),   # in place on o likewise
    (dict(h=FAKE + 2), sq.ERR_ALIGN),      # then every sharq_prepare check on h and the views
    (dict(m=0), sq.ERR_SHAPE),
    (dict(sp=view(ld_codes=63)), sq.ERR_SHAPE),
    (dict(h=FAKE + 8192, ld_h=1 << 26), sq.ERR_UNSUPPORTED),   # row strides below 2^26
    (dict(o=FAKE + 8192, ld_o=1 << 26), sq.ERR_UNSUPPORTED),
    (dict(out=FAKE + 4096, ld_out=1 << 26), sq.ERR_UNSUPPORTED),
])
def test_prepare_residual_validation(kwargs, status):
    assert prep_res(**kwargs) == status


def prep_silu(fmt=0, gate=FAKE, ld_gate=256, up=FAKE, ld_up=256, m=16, k=256, sp=None, rs=None):
    sp = sp or view(ld_codes=64)
    rs = rs or view(meta=None)
    return sq.lib().sharq_prepare_silu_mul(fmt, gate, ld_gate, up, ld_up, m, k, ctypes.byref(sp),
                                           ctypes.byref(rs), None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(fmt=1), sq.ERR_UNSUPPORTED),
    (dict(fmt=7), sq.ERR_UNSUPPORTED),
    (dict(gate=None), sq.ERR_NULL),
    (dict(up=None), sq.ERR_NULL),
    (dict(m=0), sq.ERR_SHAPE),
    (dict(k=100, ld_gate=100, ld_up=100), sq.ERR_SHAPE),
    (dict(ld_gate=128), sq.ERR_SHAPE),
    (dict(ld_up=128), sq.ERR_SHAPE),
    (dict(ld_gate=258), sq.ERR_ALIGN),
    (dict(up=FAKE + 4), sq.ERR_ALIGN),
    (dict(ld_gate=1 << 26), sq.ERR_UNSUPPORTED),   # row strides below 2^26
    (dict(ld_up=1 << 26), sq.ERR_UNSUPPORTED),
    (dict(sp=view(ld_codes=63)), sq.ERR_SHAPE),
    (dict(sp=ksm(), rs=view(meta=None)), sq.ERR_SHAPE),
    (dict(rs=view(meta=None, scales=None)), sq.ERR_NULL),
])
def test_prepare_silu_mul_validation(kwargs, status):
    assert prep_silu(**kwargs) == status


NULLV = object()   # pass a NULL view pointer


def silu_gemm(fmt=0, m=16, inter=128, k=256, sp=None, rs=None, ws=None, wd=None, osp=None, ors=None):
    sp = sp or view(ld_codes=64, dense=FAKE, ld_dense=128)
    rs = rs or view(meta=None)
    ws = ws or view(meta=None)
    wd = wd or ws
    osp = osp or view(ld_codes=32, ld_meta=16, ld_scales=4)
    ors = ors or view(meta=None, ld_codes=64, ld_scales=4)
    ref = [None if v is NULLV else ctypes.byref(v) for v in (sp, rs, ws, wd, osp, ors)]
    return sq.lib().sharq_dual_gemm_silu_prepare(fmt, ref[0], ref[1], ref[2], ref[3], m, inter, k,
                                                 ref[4], ref[5], None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(fmt=1), sq.ERR_UNSUPPORTED),
    (dict(fmt=7), sq.ERR_UNSUPPORTED),
    (dict(sp=NULLV), sq.ERR_NULL),
    (dict(osp=NULLV), sq.ERR_NULL),
    (dict(ors=NULLV), sq.ERR_NULL),
    (dict(m=0), sq.ERR_SHAPE),
    (dict(inter=64), sq.ERR_SHAPE),
    (dict(inter=192), sq.ERR_SHAPE),                    # x's columns come in 128-column tiles
    (dict(k=192), sq.ERR_SHAPE),
    (dict(sp=view(ld_codes=64)), sq.ERR_UNSUPPORTED),   # no dense backbone view
    (dict(wd=view(meta=None, codes=FAKE + 4096)), sq.ERR_SHAPE),   # two payloads
    (dict(ws=view(meta=None, ld_codes=100)), sq.ERR_SHAPE),
    (dict(ws=view(meta=None, ld_scales=6)), sq.ERR_SHAPE),
    (dict(osp=view(ld_codes=31, ld_meta=16, ld_scales=4)), sq.ERR_SHAPE),
    (dict(ors=view(meta=None, ld_codes=64, scales=None)), sq.ERR_NULL),
    (dict(osp=ksm(), ors=view(meta=None, ld_codes=64, ld_scales=4)), sq.ERR_SHAPE),   # output layouts differ
    (dict(osp=ksm(8), ors=ksm(8, meta=None)), sq.ERR_SHAPE),                         # rows per step < m
])
def test_dual_gemm_silu_prepare_validation(kwargs, status):
    assert silu_gemm(**kwargs) == status


def grouped_silu(fmt=0, tokens=16, idx=FAKE, offs=FAKE, groups=2, rows=32, inter=128, k=256, sp=None, rs=None,
                 ws=None, wd=None, osp=None, ors=None):
    sp = sp or view(ld_codes=64, dense=FAKE, ld_dense=128)
    rs = rs or view(meta=None)
    ws = ws or view(meta=None)
    wd = wd or ws
    osp = osp or view(ld_codes=32, ld_meta=16, ld_scales=4)
    ors = ors or view(meta=None, ld_codes=64, ld_scales=4)
    ref = [None if v is NULLV else ctypes.byref(v) for v in (sp, rs, ws, wd, osp, ors)]
    return sq.lib().sharq_grouped_dual_gemm_silu_prepare(fmt, ref[0], ref[1], tokens, idx, offs, groups, rows,
                                                         ref[2], ref[3], inter, k, ref[4], ref[5], None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(fmt=1), sq.ERR_UNSUPPORTED),
    (dict(groups=0), sq.ERR_UNSUPPORTED),
    (dict(groups=257), sq.ERR_UNSUPPORTED),
    (dict(offs=None), sq.ERR_NULL),
    (dict(osp=NULLV), sq.ERR_NULL),
    (dict(tokens=0), sq.ERR_SHAPE),
    (dict(rows=-1), sq.ERR_SHAPE),
    (dict(inter=192), sq.ERR_SHAPE),
    (dict(k=192), sq.ERR_SHAPE),
    (dict(idx=None, rows=17), sq.ERR_SHAPE),
    (dict(offs=FAKE + 4), sq.ERR_ALIGN),
    (dict(sp=view(ld_codes=64)), sq.ERR_UNSUPPORTED),   # no dense backbone view
    (dict(wd=view(meta=None, codes=FAKE + 4096)), sq.ERR_SHAPE),
    (dict(osp=view(ld_codes=31, ld_meta=16, ld_scales=4)), sq.ERR_SHAPE),
    (dict(osp=ksm(16), ors=ksm(16, meta=None)), sq.ERR_SHAPE),   # rows per step < rows (32)
    (dict(rows=0), sq.OK),                                       # nothing to do: no launch
])
def test_grouped_dual_gemm_silu_prepare_validation(kwargs, status):
    assert grouped_silu(**kwargs) == status


def grouped(fmt=0, tokens=16, idx=FAKE, offs=FAKE, groups=2, rows=32, n=256, k=256, y=FAKE,
            ld_y=256, sp=None, rs=None, ws=None, wd=None):
    sp = sp or view(ld_codes=64, dense=FAKE, ld_dense=128)
    rs = rs or view(meta=None)
    ws = ws or view(meta=None)
    wd = wd or ws
    return sq.lib().sharq_grouped_dual_gemm(fmt, ctypes.byref(sp), ctypes.byref(rs), tokens, idx, offs,
                                            groups, rows, ctypes.byref(ws), ctypes.byref(wd), n, k, y,
                                            ld_y, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(fmt=1), sq.ERR_UNSUPPORTED),
    (dict(groups=0), sq.ERR_UNSUPPORTED),
    (dict(groups=257), sq.ERR_UNSUPPORTED),
    (dict(offs=None), sq.ERR_NULL),
    (dict(y=None), sq.ERR_NULL),
    (dict(tokens=0), sq.ERR_SHAPE),
    (dict(rows=-1), sq.ERR_SHAPE),
    (dict(k=192), sq.ERR_SHAPE),
    (dict(ld_y=100), sq.ERR_SHAPE),
    (dict(idx=None, rows=17), sq.ERR_SHAPE),            # identity gather past the last token
    (dict(offs=FAKE + 4), sq.ERR_ALIGN),
    (dict(idx=FAKE + 2), sq.ERR_ALIGN),
    (dict(y=FAKE + 2), sq.ERR_ALIGN),
    (dict(sp=view(ld_codes=64)), sq.ERR_UNSUPPORTED),   # no dense backbone view
    (dict(wd=view(meta=None, codes=FAKE + 4096)), sq.ERR_SHAPE),   # two payloads
    (dict(ws=view(meta=None, ld_codes=100)), sq.ERR_SHAPE),
])
def test_grouped_dual_gemm_validation(kwargs, status):
    assert grouped(**kwargs) == status


def gemm(fmt=0, m=16, n=256, k=256, y=FAKE, ld_y=256, variant=0, sp=None, rs=None, ws=None,
         wd=None):
    sp = sp or view(ld_codes=64)
    rs = rs or view(meta=None)
    ws = ws or view(meta=None)
    wd = wd or view(meta=None)
    return sq.lib().sharq_dual_gemm(fmt, ctypes.byref(sp), ctypes.byref(rs), ctypes.byref(ws),
                                    ctypes.byref(wd), m, n, k, y, ld_y, variant, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(y=None), sq.ERR_NULL),
    (dict(k=192), sq.ERR_SHAPE),
    (dict(n=0), sq.ERR_SHAPE),
    (dict(ld_y=100), sq.ERR_SHAPE),
    (dict(wd=view(meta=None, codes=FAKE + 4096)), sq.ERR_SHAPE),   # two payloads
    (dict(variant=sq.GEMM_SPARSE_MFMA, sp=view(ld_codes=64, meta=None)), sq.ERR_NULL),   # reads the 2:4 form
    (dict(variant=9), sq.ERR_UNSUPPORTED),
    (dict(variant=sq.GEMM_DENSE_EXPANDED), sq.ERR_NULL),
    (dict(rs=view(meta=None, scales=FAKE + 2)), sq.ERR_ALIGN),
    (dict(sp=view(ld_codes=64, ld_scales=6)), sq.ERR_SHAPE),
    (dict(sp=view(ld_codes=72)), sq.ERR_ALIGN),
    (dict(y=FAKE + 1), sq.ERR_ALIGN),
    (dict(fmt=1), sq.ERR_SHAPE),      # NVFP4 needs k/16 scales per row (ld 8 < 16)
    (dict(ws=ksm(256, meta=None), wd=view(meta=None)), sq.ERR_SHAPE),   # W views' layouts differ
    (dict(sp=ksm(8), rs=ksm(meta=None), ws=ksm(256, meta=None), wd=ksm(256, meta=None)),
     sq.ERR_SHAPE),                   # rows per step < m
    (dict(sp=ksm(scales=FAKE + 2), rs=ksm(meta=None), ws=ksm(256, meta=None), wd=ksm(256, meta=None)),
     sq.ERR_ALIGN),
])
def test_gemm_validation(kwargs, status):
    assert gemm(**kwargs) == status


def gemm_bf16(fmt=0, m=16, n=256, k=256, y=FAKE, ld_y=256, variant=0):
    sp, rs, ws, wd = view(ld_codes=64), view(meta=None), view(meta=None), view(meta=None)
    return sq.lib().sharq_dual_gemm_bf16(fmt, ctypes.byref(sp), ctypes.byref(rs), ctypes.byref(ws),
                                         ctypes.byref(wd), m, n, k, y, ld_y, variant, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(y=None), sq.ERR_NULL),
    (dict(y=FAKE + 1), sq.ERR_ALIGN),        # bf16 output: 2-byte alignment
    (dict(ld_y=255), sq.ERR_SHAPE),
    (dict(k=192), sq.ERR_SHAPE),
    (dict(variant=9), sq.ERR_UNSUPPORTED),
    (dict(fmt=1), sq.ERR_SHAPE),
])
def test_gemm_bf16_validation(kwargs, status):
    assert gemm_bf16(**kwargs) == status


def test_gemm_bf16_output_alignment_is_two_bytes():
    """A 2-byte aligned bf16 output passes the output checks (the call then
    fails on the views: m = 0 rows, refused before any launch)."""
    assert gemm_bf16(y=FAKE + 2, m=0) == sq.ERR_SHAPE
    assert gemm(y=FAKE + 2) == sq.ERR_ALIGN


def test_quantize_weight_validation():
    L = sq.lib()
    v = view(meta=None)
    assert L.sharq_quantize_weight(0, None, 16, 256, 256, ctypes.byref(v), None) == sq.ERR_NULL
    assert L.sharq_quantize_weight(0, FAKE, 16, 48, 48, ctypes.byref(v), None) == sq.ERR_SHAPE
    assert L.sharq_quantize_weight(0, FAKE, 0, 256, 256, ctypes.byref(v), None) == sq.ERR_SHAPE
    assert L.sharq_quantize_weight(0, FAKE + 4, 16, 256, 256, ctypes.byref(v), None) == sq.ERR_ALIGN
    nv = view(meta=None, ld_scales=16)
    assert L.sharq_quantize_weight(1, FAKE, 16, 256, 256, ctypes.byref(nv), None) == sq.ERR_NULL
    k1 = ksm(meta=None, codes=FAKE + 8)
    assert L.sharq_quantize_weight(0, FAKE, 16, 256, 256, ctypes.byref(k1), None) == sq.ERR_ALIGN
    k2 = ksm(meta=None)
    assert L.sharq_quantize_weight(0, FAKE, 16, 160, 160, ctypes.byref(k2), None) == sq.ERR_SHAPE


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(sq, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(sq, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        sq.lib()


def test_binding_refuses_strided_rows():
    """The library reads and writes each row as contiguous elements: a view
    whose last dimension is strided (x[:, ::2]) must be refused by the
    binding, not passed on with a row stride that the ABI would accept."""
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    assert sq._ld(x) == 64
    assert sq._ld(x[:, :32]) == 64          # padded rows are fine
    assert sq._ld(x[:1]) == 64
    for bad in (x[:, ::2], x.t(), x.view(4, 8, 8)):
        with pytest.raises(ValueError):
            sq._ld(bad)


def test_dual_gemm_output_dtype_checks():
    """The binding refuses an output type other than fp32 or bf16, and an
    `out` whose type contradicts out_dtype, before any library call."""
    import torch
    with pytest.raises(TypeError, match="out_dtype"):
        sq.dual_gemm(None, None, None, out_dtype=torch.float16)
    with pytest.raises(TypeError, match="out is"):
        sq.dual_gemm(None, None, None, out=torch.empty(2, 2), out_dtype=torch.bfloat16)
