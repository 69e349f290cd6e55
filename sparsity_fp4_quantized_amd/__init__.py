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

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsharq.so")

# every symbol include/sharq.h declares
EXPORTS = ("sharq_quantize_weight", "sharq_prepare", "sharq_dual_gemm", "sharq_bytes",
           "sharq_status_str", "sharq_abi_version")
ABI_VERSION = 1


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
        L.sharq_dual_gemm.argtypes = [ctypes.c_int, V, V, V, V, I64, I64, I64, P, I64,
                                      ctypes.c_int, P]
        L.sharq_dual_gemm.restype = ctypes.c_int
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


def _bits16(t):
    """bf16 (or int16/uint16 bit pattern) tensor -> its data, as stored."""
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected a bfloat16 tensor (or its 16-bit pattern), got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError("tensor must be on the GPU")
    return t


@dataclasses.dataclass
class FP4Tensor:
    """Device buffers of one FP4 operand (see ``sharq_fp4_view``)."""
    fmt: int
    rows: int
    k: int
    codes: object                   # uint8 [rows, k/2] or [rows, k/4] (backbone)
    scales: object                  # uint8 [rows, k/blk]
    meta: object = None             # uint8 [rows, k/8] (backbone)
    dense_codes: object = None      # uint8 [rows, k/2] (optional backbone view)
    tensor_scale: object = None     # float32 [2] (NVFP4)

    def view(self) -> FP4ViewC:
        v = FP4ViewC()
        v.codes = _ptr(self.codes)
        v.ld_codes = self.codes.stride(0)
        if self.meta is not None:
            v.meta = _ptr(self.meta)
            v.ld_meta = self.meta.stride(0)
        v.scales = _ptr(self.scales)
        v.ld_scales = self.scales.stride(0)
        if self.dense_codes is not None:
            v.dense_codes = _ptr(self.dense_codes)
            v.ld_dense = self.dense_codes.stride(0)
        if self.tensor_scale is not None:
            v.tensor_scale = _ptr(self.tensor_scale)
        return v


def _alloc(rows, cols, device, dtype=None):
    torch = _torch()
    return torch.empty((rows, cols), dtype=dtype or torch.uint8, device=device)


def quantize_weight(w, fmt: int = MXFP4, stream=None) -> FP4Tensor:
    """One FP4 payload of W [n, k] (both GEMM paths read it)."""
    torch = _torch()
    w = _bits16(w)
    n, k = w.shape
    blk = BLOCK[fmt]
    out = FP4Tensor(fmt, n, k, _alloc(n, k // 2, w.device), _alloc(n, k // blk, w.device))
    if fmt == NVFP4:
        out.tensor_scale = torch.zeros(2, dtype=torch.float32, device=w.device)
    v = out.view()
    _check(lib().sharq_quantize_weight(fmt, w.data_ptr(), n, k, w.stride(0), ctypes.byref(v),
                                       _stream_ptr(stream)), "sharq_quantize_weight")
    return out


def prepare(x, gamma=None, eps: float = 1e-5, fmt: int = MXFP4, dense_backbone: bool = False,
            stream=None):
    """Fused preparation of X [m, k]: returns (backbone, residual) FP4 operands."""
    torch = _torch()
    x = _bits16(x)
    m, k = x.shape
    blk = BLOCK[fmt]
    dev = x.device
    sp = FP4Tensor(fmt, m, k, _alloc(m, k // 4, dev), _alloc(m, k // blk, dev),
                   meta=_alloc(m, k // 8, dev))
    if dense_backbone:
        sp.dense_codes = _alloc(m, k // 2, dev)
    rs = FP4Tensor(fmt, m, k, _alloc(m, k // 2, dev), _alloc(m, k // blk, dev))
    if fmt == NVFP4:
        sp.tensor_scale = torch.zeros(2, dtype=torch.float32, device=dev)
        rs.tensor_scale = sp.tensor_scale
    prepare_into(x, gamma, eps, sp, rs, stream)
    return sp, rs


def prepare_into(x, gamma, eps, sp: FP4Tensor, rs: FP4Tensor, stream=None):
    """sharq_prepare into caller-provided buffers (nothing is allocated)."""
    x = _bits16(x)
    g = None if gamma is None else _bits16(gamma)
    m, k = x.shape
    vs, vr = sp.view(), rs.view()
    _check(lib().sharq_prepare(sp.fmt, x.data_ptr(), m, k, x.stride(0), _ptr(g), float(eps),
                               ctypes.byref(vs), ctypes.byref(vr), _stream_ptr(stream)),
           "sharq_prepare")


def dual_gemm(sp: FP4Tensor, rs: FP4Tensor, w: FP4Tensor, variant: int = GEMM_AUTO,
              w_dense_scales=None, out=None, stream=None):
    """Y = deq(backbone) deq(W)^T + deq(residual) deq(W)^T, fp32 [m, n]."""
    torch = _torch()
    m, k, n = sp.rows, sp.k, w.rows
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=w.codes.device)
    wv_s = w.view()
    wv_d = w.view()
    if w_dense_scales is not None:
        wv_d.scales = _ptr(w_dense_scales)
        wv_d.ld_scales = w_dense_scales.stride(0)
    vs, vr = sp.view(), rs.view()
    _check(lib().sharq_dual_gemm(sp.fmt, ctypes.byref(vs), ctypes.byref(vr), ctypes.byref(wv_s),
                                 ctypes.byref(wv_d), m, n, k, out.data_ptr(), out.stride(0),
                                 variant, _stream_ptr(stream)), "sharq_dual_gemm")
    return out
