"""SharQ linear-layer hot path for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/sharq.h`` (``libsharq.so``,
built in-tree by ``sparsity_fp4_quantized_amd/build.py``).  The binding only
marshals arguments: torch provides device memory and the current HIP
stream, and every step of the path runs in the library's HIP kernels.  There
is no CPU fallback: without the built library every call raises.

Method: "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
Inference" (arXiv:2606.26587), abstract, sentences 3-5 and 7.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

MXFP4 = 0
NVFP4 = 1
BLOCK = {MXFP4: 32, NVFP4: 16}

GEMM_AUTO = 0
GEMM_DECOMPRESS = 1
GEMM_DENSE_EXPANDED = 2
GEMM_SPARSE_MFMA = 3

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_DEVICE = range(6)

BYTES_DENSE_CODES, BYTES_SPARSE_CODES, BYTES_META, BYTES_SCALES = range(4)

LAYOUT_ROW_MAJOR = 0
LAYOUT_KSTEP_MAJOR = 1

# bytes per row and 128-k step of each array of an operand (k-step-major layout)
BPS_CODES, BPS_SPARSE_CODES, BPS_META = 64, 32, 16

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsharq.so")

# every symbol include/sharq.h declares
EXPORTS = ("sharq_quantize_weight", "sharq_prepare", "sharq_prepare_residual", "sharq_prepare_silu_mul",
           "sharq_dual_gemm", "sharq_dual_gemm_silu_prepare", "sharq_grouped_dual_gemm",
           "sharq_grouped_dual_gemm_silu_prepare", "sharq_bytes", "sharq_status_str", "sharq_abi_version",
           "sharq_prepare_noalloc", "sharq_dual_gemm_bf16")
ABI_VERSION = 11


class SharqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class FP4ViewC(ctypes.Structure):
    """Mirror of ``sharq_fp4_view``."""
    _fields_ = [
        ("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
        ("meta", ctypes.c_void_p), ("ld_meta", ctypes.c_int64),
        ("scales", ctypes.c_void_p), ("ld_scales", ctypes.c_int64),
        ("layout", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("dense_codes", ctypes.c_void_p), ("ld_dense", ctypes.c_int64),
        ("tensor_scale", ctypes.c_void_p),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python sparsity_fp4_quantized_amd/build.py` "
                "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        V = ctypes.POINTER(FP4ViewC)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.sharq_quantize_weight.argtypes = [ctypes.c_int, P, I64, I64, I64, V, P]
        L.sharq_quantize_weight.restype = ctypes.c_int
        L.sharq_prepare.argtypes = [ctypes.c_int, P, I64, I64, I64, P, ctypes.c_float, V, V, P]
        L.sharq_prepare.restype = ctypes.c_int
        L.sharq_prepare_noalloc.argtypes = [ctypes.c_int, P, I64, I64, I64, P, ctypes.c_float, V, V, P]
        L.sharq_prepare_noalloc.restype = ctypes.c_int
        L.sharq_prepare_residual.argtypes = [ctypes.c_int, P, I64, P, I64, P, I64, I64, I64, P,
                                             ctypes.c_float, V, V, P]
        L.sharq_prepare_residual.restype = ctypes.c_int
        L.sharq_prepare_silu_mul.argtypes = [ctypes.c_int, P, I64, P, I64, I64, I64, V, V, P]
        L.sharq_prepare_silu_mul.restype = ctypes.c_int
        L.sharq_dual_gemm_silu_prepare.argtypes = [ctypes.c_int, V, V, V, V, I64, I64, I64, V, V, P]
        L.sharq_dual_gemm_silu_prepare.restype = ctypes.c_int
        L.sharq_grouped_dual_gemm_silu_prepare.argtypes = [ctypes.c_int, V, V, I64, P, P, I64, I64, V, V,
                                                           I64, I64, V, V, P]
        L.sharq_grouped_dual_gemm_silu_prepare.restype = ctypes.c_int
        L.sharq_grouped_dual_gemm.argtypes = [ctypes.c_int, V, V, I64, P, P, I64, I64, V, V, I64, I64,
                                              P, I64, P]
        L.sharq_grouped_dual_gemm.restype = ctypes.c_int
        L.sharq_dual_gemm.argtypes = [ctypes.c_int, V, V, V, V, I64, I64, I64, P, I64,
                                      ctypes.c_int, P]
        L.sharq_dual_gemm.restype = ctypes.c_int
        L.sharq_dual_gemm_bf16.argtypes = [ctypes.c_int, V, V, V, V, I64, I64, I64, P, I64,
                                           ctypes.c_int, P]
        L.sharq_dual_gemm_bf16.restype = ctypes.c_int
        L.sharq_bytes.argtypes = [ctypes.c_int, ctypes.c_int, I64, I64]
        L.sharq_bytes.restype = ctypes.c_size_t
        L.sharq_status_str.argtypes = [ctypes.c_int]
        L.sharq_status_str.restype = ctypes.c_char_p
        L.sharq_abi_version.argtypes = []
        L.sharq_abi_version.restype = ctypes.c_int
        if L.sharq_abi_version() != ABI_VERSION:
            raise RuntimeError("libsharq.so ABI version mismatch; rebuild it")
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().sharq_status_str(int(status)).decode()


def nbytes(fmt: int, which: int, rows: int, k: int) -> int:
    return int(lib().sharq_bytes(fmt, which, rows, k))


def _check(status: int, where: str):
    if status != OK:
        raise SharqError(status, where)


# ------------------------------------------------------------------ torch side
def _torch():
    import torch
    return torch


def _stream_ptr(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _ld(t) -> int:
    """Row stride of a row-major 2-D tensor, in elements (the stride of a
    single-row tensor is arbitrary; its row length is used instead).  The
    library reads and writes each row as contiguous elements, so a view whose
    last dimension is strided is refused."""
    if t.dim() != 2:
        raise ValueError(f"expected a 2-D tensor, got {t.dim()} dimensions")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("the last dimension must have unit stride (rows are read as contiguous elements)")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _vec(t, n: int, what: str):
    """A 1-D device tensor of n contiguous elements."""
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on the GPU")
    if t.dim() != 1 or t.shape[0] != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{what} must be a contiguous 1-D tensor of {n} elements")
    return t


def _bits16(t):
    """bf16 (or int16/uint16 bit pattern) tensor -> its data, as stored."""
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected a bfloat16 tensor (or its 16-bit pattern), got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError("tensor must be on the GPU")
    return t


def scale_bps(fmt: int) -> int:
    """Scale bytes per row and 128-k step."""
    return 128 // BLOCK[fmt]


def _ld_of(t, layout: int, bps: int) -> int:
    """ld of one array: bytes per row (row-major) or rows per step (k-step-major)."""
    if layout == LAYOUT_KSTEP_MAJOR:
        if t.dim() != 3 or t.shape[2] != bps or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != bps):
            raise ValueError(f"k-step-major array must be [k/128, rows, {bps}], contiguous within a step")
        return t.stride(0) // bps if t.shape[0] > 1 else t.shape[1]
    return _ld(t)


@dataclasses.dataclass
class FP4Tensor:
    """Device buffers of one FP4 operand (see ``sharq_fp4_view``).

    Every array is in ``layout``: row-major [rows, bytes per row], or
    k-step-major [k/128, rows, bytes per row and step] (codes 64, 2:4 codes
    32, meta 16, scales 4 (MXFP4) or 8 (NVFP4)), the layout the GEMM streams
    fastest.  ``codes`` is 2:4-compressed when ``meta`` is set."""
    fmt: int
    rows: int
    k: int
    codes: object
    scales: object
    meta: object = None             # 2:4 indices (backbone)
    dense_codes: object = None      # optional dense backbone view
    tensor_scale: object = None     # float32 [2] (NVFP4)
    layout: int = LAYOUT_ROW_MAJOR

    def __setattr__(self, name, value):
        # any change of a field drops the cached C view
        object.__setattr__(self, "_vc", None)
        object.__setattr__(self, name, value)

    def view(self) -> FP4ViewC:
        """The C view (built once, then cached until a field changes)."""
        vc = getattr(self, "_vc", None)
        if vc is None:
            vc = self._build_view()
            object.__setattr__(self, "_vc", vc)
        return vc

    def _build_view(self) -> FP4ViewC:
        v = FP4ViewC()
        L = self.layout
        v.layout = L
        v.codes = _ptr(self.codes)
        v.ld_codes = _ld_of(self.codes, L, BPS_SPARSE_CODES if self.meta is not None else BPS_CODES)
        if self.meta is not None:
            v.meta = _ptr(self.meta)
            v.ld_meta = _ld_of(self.meta, L, BPS_META)
        v.scales = _ptr(self.scales)
        v.ld_scales = _ld_of(self.scales, L, scale_bps(self.fmt))
        if self.dense_codes is not None:
            v.dense_codes = _ptr(self.dense_codes)
            v.ld_dense = _ld_of(self.dense_codes, L, BPS_CODES)
        if self.tensor_scale is not None:
            v.tensor_scale = _ptr(self.tensor_scale)
        return v

    def row_major(self, name: str):
        """Array `name` as a [rows, bytes per row] tensor (a copy if k-step-major)."""
        return row_major(getattr(self, name), self.layout, self.rows)


def row_major(arr, layout: int, rows: int):
    if layout == LAYOUT_KSTEP_MAJOR:
        return arr.permute(1, 0, 2)[:rows].reshape(rows, -1)
    return arr


def default_layout(k: int) -> int:
    return LAYOUT_KSTEP_MAJOR if k % 128 == 0 else LAYOUT_ROW_MAJOR


def alloc_array(rows: int, k: int, bps: int, layout: int, device):
    """Uninitialized array of `rows` rows with `bps` bytes per row and 128-k step."""
    torch = _torch()
    if layout == LAYOUT_KSTEP_MAJOR:
        return torch.empty((k // 128, rows, bps), dtype=torch.uint8, device=device)
    return torch.empty((rows, k * bps // 128), dtype=torch.uint8, device=device)


def alloc_scales(fmt: int, rows: int, k: int, layout: int, device):
    return alloc_array(rows, k, scale_bps(fmt), layout, device)


def scales_row_major(t: FP4Tensor):
    """The operand's scales as a [rows, k/blk] tensor (a copy if k-step-major)."""
    return t.row_major("scales")


def quantize_weight(w, fmt: int = MXFP4, layout: Optional[int] = None, stream=None) -> FP4Tensor:
    """One FP4 payload of W [n, k] (both GEMM paths read it)."""
    torch = _torch()
    w = _bits16(w)
    n, k = w.shape
    L = default_layout(k) if layout is None else layout
    out = FP4Tensor(fmt, n, k, alloc_array(n, k, BPS_CODES, L, w.device),
                    alloc_scales(fmt, n, k, L, w.device), layout=L)
    if fmt == NVFP4:
        out.tensor_scale = torch.zeros(2, dtype=torch.float32, device=w.device)
    v = out.view()
    _check(lib().sharq_quantize_weight(fmt, w.data_ptr(), n, k, _ld(w), ctypes.byref(v),
                                       _stream_ptr(stream)), "sharq_quantize_weight")
    return out


def alloc_prepared(fmt: int, m: int, k: int, device, dense_backbone: bool = False,
                   layout: Optional[int] = None):
    """Uninitialized (backbone, residual) operands for sharq_prepare."""
    torch = _torch()
    L = default_layout(k) if layout is None else layout
    sp = FP4Tensor(fmt, m, k, alloc_array(m, k, BPS_SPARSE_CODES, L, device),
                   alloc_scales(fmt, m, k, L, device), meta=alloc_array(m, k, BPS_META, L, device),
                   layout=L)
    if dense_backbone:
        sp.dense_codes = alloc_array(m, k, BPS_CODES, L, device)
    rs = FP4Tensor(fmt, m, k, alloc_array(m, k, BPS_CODES, L, device),
                   alloc_scales(fmt, m, k, L, device), layout=L)
    if fmt == NVFP4:
        sp.tensor_scale = torch.zeros(2, dtype=torch.float32, device=device)
        rs.tensor_scale = sp.tensor_scale
    return sp, rs


def prepare(x, gamma=None, eps: float = 1e-5, fmt: int = MXFP4, dense_backbone: bool = False,
            layout: Optional[int] = None, stream=None):
    """Fused preparation of X [m, k]: returns (backbone, residual) FP4 operands."""
    x = _bits16(x)
    m, k = x.shape
    sp, rs = alloc_prepared(fmt, m, k, x.device, dense_backbone, layout)
    prepare_into(x, gamma, eps, sp, rs, stream)
    return sp, rs


class BoundCall:
    """One library call with its arguments marshalled once (pointers, sizes,
    views and the stream, taken when it is bound): calling it only crosses into
    the library, which launches the kernels.  For loops that run the same
    buffers again and again; the tensors it was bound to must stay alive and
    keep their storage."""
    __slots__ = ("_fn", "_args", "_where", "_keep")

    def __init__(self, fn, args, where, keep):
        self._fn, self._args, self._where, self._keep = fn, args, where, keep

    def __call__(self):
        status = self._fn(*self._args)
        if status != OK:
            raise SharqError(status, self._where)


def bind_prepare(x, gamma, eps, sp: FP4Tensor, rs: FP4Tensor, stream=None, noalloc: bool = False) -> BoundCall:
    """sharq_prepare (or, noalloc, sharq_prepare_noalloc) into caller-provided
    buffers, bound for repeated calls."""
    x = _bits16(x)
    m, k = x.shape
    g = None if gamma is None else _vec(_bits16(gamma), k, "gamma")
    vs, vr = sp.view(), rs.view()
    args = (ctypes.c_int(sp.fmt), ctypes.c_void_p(x.data_ptr()), ctypes.c_int64(m), ctypes.c_int64(k),
            ctypes.c_int64(_ld(x)), ctypes.c_void_p(_ptr(g)), ctypes.c_float(float(eps)),
            ctypes.byref(vs), ctypes.byref(vr), _stream_ptr(stream))
    fn, where = (lib().sharq_prepare_noalloc, "sharq_prepare_noalloc") if noalloc else (lib().sharq_prepare, "sharq_prepare")
    return BoundCall(fn, args, where, (x, g, sp, rs, vs, vr))


def prepare_into(x, gamma, eps, sp: FP4Tensor, rs: FP4Tensor, stream=None):
    """sharq_prepare into caller-provided buffers (nothing is allocated)."""
    bind_prepare(x, gamma, eps, sp, rs, stream)()


def bind_prepare_residual(h, o, gamma, eps, sp: FP4Tensor, rs: FP4Tensor, out, stream=None) -> BoundCall:
    """sharq_prepare_residual: out = bf16(h + o) (the new residual stream; may
    be h or o itself), then the preparation of out, bound for repeated calls."""
    h, o, out = _bits16(h), _bits16(o), _bits16(out)
    m, k = h.shape
    g = _vec(_bits16(gamma), k, "gamma")
    if tuple(o.shape) != (m, k) or tuple(out.shape) != (m, k):
        raise ValueError("h, o and out must have the same shape")
    vs, vr = sp.view(), rs.view()
    args = (ctypes.c_int(sp.fmt), ctypes.c_void_p(h.data_ptr()), ctypes.c_int64(_ld(h)),
            ctypes.c_void_p(o.data_ptr()), ctypes.c_int64(_ld(o)), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_int64(_ld(out)), ctypes.c_int64(m), ctypes.c_int64(k), ctypes.c_void_p(g.data_ptr()),
            ctypes.c_float(float(eps)), ctypes.byref(vs), ctypes.byref(vr), _stream_ptr(stream))
    return BoundCall(lib().sharq_prepare_residual, args, "sharq_prepare_residual",
                     (h, o, out, g, sp, rs, vs, vr))


def prepare_residual(h, o, gamma, eps: float = 1e-5, dense_backbone: bool = False,
                     layout: Optional[int] = None, out=None, stream=None):
    """Residual add fused into the preparation (MXFP4): returns (x, backbone,
    residual) with x = bf16(h + o) written to `out` (a new tensor when None;
    pass h to update the residual stream in place)."""
    torch = _torch()
    h = _bits16(h)
    m, k = h.shape
    if out is None:
        out = torch.empty_like(h)
    sp, rs = alloc_prepared(MXFP4, m, k, h.device, dense_backbone, layout)
    bind_prepare_residual(h, o, gamma, eps, sp, rs, out, stream)()
    return out, sp, rs


def _f32(t):
    torch = _torch()
    if t.dtype != torch.float32:
        raise TypeError(f"expected a float32 tensor, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError("tensor must be on the GPU")
    return t


def bind_prepare_silu_mul(gate, up, sp: FP4Tensor, rs: FP4Tensor, stream=None) -> BoundCall:
    """sharq_prepare_silu_mul: the preparation (no norm) of x = bf16(silu(gate)
    * up), from fp32 gate and up [m, k], bound for repeated calls."""
    gate, up = _f32(gate), _f32(up)
    m, k = gate.shape
    if tuple(up.shape) != (m, k):
        raise ValueError("gate and up must have the same shape")
    vs, vr = sp.view(), rs.view()
    args = (ctypes.c_int(sp.fmt), ctypes.c_void_p(gate.data_ptr()), ctypes.c_int64(_ld(gate)),
            ctypes.c_void_p(up.data_ptr()), ctypes.c_int64(_ld(up)), ctypes.c_int64(m), ctypes.c_int64(k),
            ctypes.byref(vs), ctypes.byref(vr), _stream_ptr(stream))
    return BoundCall(lib().sharq_prepare_silu_mul, args, "sharq_prepare_silu_mul", (gate, up, sp, rs, vs, vr))


def prepare_silu_mul(gate, up, dense_backbone: bool = False, layout: Optional[int] = None, stream=None):
    """SiLU(gate) * up fused into the preparation (MXFP4, no norm): returns the
    (backbone, residual) operands of the down projection.  gate and up may be
    the two column halves of the gate+up projection's fp32 output."""
    m, k = gate.shape
    sp, rs = alloc_prepared(MXFP4, m, k, gate.device, dense_backbone, layout)
    bind_prepare_silu_mul(gate, up, sp, rs, stream)()
    return sp, rs


def bind_dual_gemm(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, out, variant: int = GEMM_AUTO,
                   w_dense_scales=None, stream=None) -> BoundCall:
    """sharq_dual_gemm into `out` (fp32 [m, n]), or sharq_dual_gemm_bf16 when
    `out` is bfloat16, bound for repeated calls."""
    m, k, n = sp.rows, sp.k, w.rows
    torch = _torch()
    bf16_out = out.dtype == torch.bfloat16
    out = _bits16(out) if bf16_out else _f32(out)
    if out.dim() != 2 or tuple(out.shape) != (m, n):
        raise ValueError(f"out must be [{m}, {n}]")
    wv_s = w.view()
    if w_dense_scales is not None:
        wv_d = FP4ViewC.from_buffer_copy(wv_s)
        wv_d.scales = _ptr(w_dense_scales)
        wv_d.ld_scales = _ld_of(w_dense_scales, w.layout, scale_bps(w.fmt))
    else:
        wv_d = wv_s
    vs, vr = sp.view(), rs.view()
    args = (ctypes.c_int(sp.fmt), ctypes.byref(vs), ctypes.byref(vr), ctypes.byref(wv_s), ctypes.byref(wv_d),
            ctypes.c_int64(m), ctypes.c_int64(n), ctypes.c_int64(k), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_int64(_ld(out)), ctypes.c_int(variant), _stream_ptr(stream))
    name = "sharq_dual_gemm_bf16" if bf16_out else "sharq_dual_gemm"
    return BoundCall(getattr(lib(), name), args, name, (sp, rs, w, out, w_dense_scales, vs, vr, wv_s, wv_d))


def dual_gemm(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, variant: int = GEMM_AUTO,
              w_dense_scales=None, out=None, stream=None, out_dtype=None):
    """Y = deq(backbone) deq(W)^T + deq(residual) deq(W)^T, [m, n]: fp32, or
    bf16 (each fp32 value rounded to nearest even) when out_dtype or `out`
    is torch.bfloat16."""
    torch = _torch()
    if out is not None and out_dtype is not None and out.dtype != out_dtype:
        raise TypeError(f"out is {out.dtype} but out_dtype is {out_dtype}")
    if out is None:
        dt = torch.float32 if out_dtype is None else out_dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise TypeError(f"out_dtype must be float32 or bfloat16, got {dt}")
        out = torch.empty((sp.rows, w.rows), dtype=dt, device=w.codes.device)
    bind_dual_gemm(sp, rs, w, out, variant, w_dense_scales, stream)()
    return out


def bind_dual_gemm_silu_prepare(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, out_sp: FP4Tensor,
                                out_rs: FP4Tensor, stream=None) -> BoundCall:
    """sharq_dual_gemm_silu_prepare: the gate+up dual GEMM (W: inter gate rows,
    then inter up rows) with x = bf16(silu(gate) * up) prepared into (out_sp,
    out_rs) [m, inter] in its epilogue, bound for repeated calls."""
    m, k = sp.rows, sp.k
    if w.rows % 2:
        raise ValueError("the gate+up weight must have 2 * inter rows")
    inter = w.rows // 2
    ws, vs, vr, vos, vor = w.view(), sp.view(), rs.view(), out_sp.view(), out_rs.view()
    args = (ctypes.c_int(sp.fmt), ctypes.byref(vs), ctypes.byref(vr), ctypes.byref(ws), ctypes.byref(ws),
            ctypes.c_int64(m), ctypes.c_int64(inter), ctypes.c_int64(k), ctypes.byref(vos), ctypes.byref(vor),
            _stream_ptr(stream))
    return BoundCall(lib().sharq_dual_gemm_silu_prepare, args, "sharq_dual_gemm_silu_prepare",
                     (sp, rs, w, out_sp, out_rs, ws, vs, vr, vos, vor))


def dual_gemm_silu_prepare(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, dense_backbone: bool = False,
                           layout: Optional[int] = None, stream=None):
    """The gate+up projection with SiLU(gate) * up and the preparation fused
    into its epilogue (MXFP4): returns the down projection's (backbone,
    residual) operands [m, inter] without writing the fp32 product."""
    inter = w.rows // 2
    out_sp, out_rs = alloc_prepared(MXFP4, sp.rows, inter, w.codes.device, dense_backbone, layout)
    bind_dual_gemm_silu_prepare(sp, rs, w, out_sp, out_rs, stream)()
    return out_sp, out_rs


def bind_grouped_dual_gemm(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, group_offsets, rows: int, out,
                           row_index=None, stream=None) -> BoundCall:
    """sharq_grouped_dual_gemm into `out` (fp32 [rows, n]): group e's rows
    (group_offsets[e] .. group_offsets[e + 1], an int64 device tensor of
    groups + 1 entries) gather activation rows row_index[i] (int32 device
    tensor; None: row i) and meet W rows e n .. e n + n - 1, bound for repeated
    calls.  `w` stacks the groups' weights: groups * n rows."""
    torch = _torch()
    if group_offsets.dtype != torch.int64 or (row_index is not None and row_index.dtype != torch.int32):
        raise TypeError("group_offsets must be int64 and row_index int32")
    groups = group_offsets.numel() - 1
    _vec(group_offsets, groups + 1, "group_offsets")
    if row_index is not None:
        _vec(row_index, row_index.numel(), "row_index")
        if row_index.numel() < rows:
            raise ValueError("row_index must hold an entry for every grouped row")
    out = _f32(out)
    if out.dim() != 2 or out.shape[0] < rows:
        raise ValueError(f"out must be 2-D with at least {rows} rows")
    n, k = out.shape[1], sp.k
    if w.rows % groups:
        raise ValueError("the stacked weight must hold the same number of rows for every group")
    if w.rows // groups != n:
        raise ValueError("out has n columns, the stacked weight groups * n rows")
    ws, vs, vr = w.view(), sp.view(), rs.view()
    args = (ctypes.c_int(sp.fmt), ctypes.byref(vs), ctypes.byref(vr), ctypes.c_int64(sp.rows),
            ctypes.c_void_p(_ptr(row_index)), ctypes.c_void_p(group_offsets.data_ptr()),
            ctypes.c_int64(groups), ctypes.c_int64(rows), ctypes.byref(ws), ctypes.byref(ws),
            ctypes.c_int64(n), ctypes.c_int64(k), ctypes.c_void_p(out.data_ptr()), ctypes.c_int64(_ld(out)),
            _stream_ptr(stream))
    return BoundCall(lib().sharq_grouped_dual_gemm, args, "sharq_grouped_dual_gemm",
                     (sp, rs, w, group_offsets, row_index, out, ws, vs, vr))


def grouped_dual_gemm(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, group_offsets, rows: int,
                      row_index=None, out=None, stream=None):
    """Grouped dual GEMM (mixture-of-experts expert GEMMs): returns Y [rows, n]."""
    torch = _torch()
    groups = group_offsets.numel() - 1
    if out is None:
        out = torch.empty((rows, w.rows // groups), dtype=torch.float32, device=w.codes.device)
    bind_grouped_dual_gemm(sp, rs, w, group_offsets, rows, out, row_index, stream)()
    return out


def bind_grouped_dual_gemm_silu_prepare(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, group_offsets, rows: int,
                                        out_sp: FP4Tensor, out_rs: FP4Tensor, row_index=None,
                                        stream=None) -> BoundCall:
    """sharq_grouped_dual_gemm_silu_prepare: every group's gate+up dual GEMM
    (group e's weight: rows e 2 inter .. of the stacked payload, inter gate
    rows then inter up rows) over its gathered rows, with x = bf16(silu(gate) *
    up) prepared into (out_sp, out_rs) [rows, inter], bound for repeated calls."""
    torch = _torch()
    if group_offsets.dtype != torch.int64 or (row_index is not None and row_index.dtype != torch.int32):
        raise TypeError("group_offsets must be int64 and row_index int32")
    groups = group_offsets.numel() - 1
    _vec(group_offsets, groups + 1, "group_offsets")
    if row_index is not None:
        _vec(row_index, row_index.numel(), "row_index")
        if row_index.numel() < rows:
            raise ValueError("row_index must hold an entry for every grouped row")
    if w.rows % (2 * groups):
        raise ValueError("the stacked weight must hold 2 * inter rows for every group")
    inter, k = w.rows // (2 * groups), sp.k
    ws, vs, vr, vos, vor = w.view(), sp.view(), rs.view(), out_sp.view(), out_rs.view()
    args = (ctypes.c_int(sp.fmt), ctypes.byref(vs), ctypes.byref(vr), ctypes.c_int64(sp.rows),
            ctypes.c_void_p(_ptr(row_index)), ctypes.c_void_p(group_offsets.data_ptr()),
            ctypes.c_int64(groups), ctypes.c_int64(rows), ctypes.byref(ws), ctypes.byref(ws),
            ctypes.c_int64(inter), ctypes.c_int64(k), ctypes.byref(vos), ctypes.byref(vor), _stream_ptr(stream))
    return BoundCall(lib().sharq_grouped_dual_gemm_silu_prepare, args, "sharq_grouped_dual_gemm_silu_prepare",
                     (sp, rs, w, group_offsets, row_index, out_sp, out_rs, ws, vs, vr, vos, vor))


def grouped_dual_gemm_silu_prepare(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, group_offsets, rows: int,
                                   row_index=None, dense_backbone: bool = False, layout: Optional[int] = None,
                                   stream=None):
    """A mixture-of-experts layer's gate+up expert GEMMs with SiLU(gate) * up
    and the down projections' preparation fused in (MXFP4): returns the
    (backbone, residual) operands [rows, inter] of the grouped rows."""
    groups = group_offsets.numel() - 1
    inter = w.rows // (2 * groups)
    out_sp, out_rs = alloc_prepared(MXFP4, max(rows, 1), inter, w.codes.device, dense_backbone, layout)
    bind_grouped_dual_gemm_silu_prepare(sp, rs, w, group_offsets, rows, out_sp, out_rs, row_index, stream)()
    return out_sp, out_rs
