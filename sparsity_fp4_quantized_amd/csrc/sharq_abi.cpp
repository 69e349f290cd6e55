// C ABI of the SharQ path: argument validation and kernel dispatch.
// Validation runs entirely on the host, before any HIP call, so that an
// invalid request enqueues nothing.
#include "../../include/sharq.h"

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace {

using sharq::GemmArgs;
using sharq::PrepArgs;
using sharq::QuantArgs;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int block_of(sharq_format f) { return f == SHARQ_MXFP4 ? 32 : 16; }

bool valid_format(sharq_format f) { return f == SHARQ_MXFP4 || f == SHARQ_NVFP4; }

sharq_status from_hip(hipError_t e) { return e == hipSuccess ? SHARQ_OK : SHARQ_ERR_DEVICE; }

// Checks of one scale array of `rows` rows.  ROW_MAJOR: [rows, k/blk] bytes;
// `dword` asks for 4-byte access (GEMM), otherwise NVFP4 needs 2-byte access
// (two blocks per lane).  KSTEP_MAJOR: ld counts rows per 128-k step.
sharq_status check_scales(sharq_format f, const sharq_fp4_view *v, int64_t rows, int64_t k,
                          bool dword) {
  if (!v->scales) return SHARQ_ERR_NULL;
  if (v->reserved != 0) return SHARQ_ERR_SHAPE;
  if (v->scale_layout == SHARQ_SCALES_KSTEP_MAJOR) {
    if (k % 128 || v->ld_scales < rows) return SHARQ_ERR_SHAPE;
    if (!aligned(v->scales, f == SHARQ_MXFP4 ? 4 : 8)) return SHARQ_ERR_ALIGN;
    return SHARQ_OK;
  }
  if (v->scale_layout != SHARQ_SCALES_ROW_MAJOR) return SHARQ_ERR_UNSUPPORTED;
  if (v->ld_scales < k / block_of(f)) return SHARQ_ERR_SHAPE;
  if (dword) {
    if (!aligned(v->scales, 4) || v->ld_scales % 4) return SHARQ_ERR_ALIGN;
  } else if (f == SHARQ_NVFP4) {
    if (!aligned(v->scales, 2) || v->ld_scales % 2) return SHARQ_ERR_ALIGN;
  }
  return SHARQ_OK;
}

int kstep(const sharq_fp4_view *v) { return v->scale_layout == SHARQ_SCALES_KSTEP_MAJOR ? 1 : 0; }

// The scale array of `rows` rows spans less than 4 GiB.
bool scales_fit(sharq_format f, const sharq_fp4_view *v, int64_t rows, int64_t k) {
  const int64_t lim = (int64_t)1 << 32;
  if (v->scale_layout == SHARQ_SCALES_KSTEP_MAJOR)
    return (k / 128) * v->ld_scales * (128 / block_of(f)) < lim;
  return rows * v->ld_scales < lim;
}

}  // namespace

extern "C" {

int sharq_abi_version(void) { return SHARQ_ABI_VERSION; }

const char *sharq_status_str(sharq_status s) {
  switch (s) {
    case SHARQ_OK: return "ok";
    case SHARQ_ERR_NULL: return "a required pointer is NULL";
    case SHARQ_ERR_SHAPE: return "invalid size, leading dimension or view pairing";
    case SHARQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case SHARQ_ERR_UNSUPPORTED: return "unsupported request";
    case SHARQ_ERR_DEVICE: return "HIP runtime error at launch";
  }
  return "unknown status";
}

size_t sharq_bytes(sharq_format f, int which, int64_t rows, int64_t k) {
  if (!valid_format(f) || rows < 0 || k <= 0 || k % 32) return 0;
  switch (which) {
    case SHARQ_BYTES_DENSE_CODES: return (size_t)(rows * (k / 2));
    case SHARQ_BYTES_SPARSE_CODES: return (size_t)(rows * (k / 4));
    case SHARQ_BYTES_META: return (size_t)(rows * (k / 8));
    case SHARQ_BYTES_SCALES: return (size_t)(rows * (k / block_of(f)));
  }
  return 0;
}

sharq_status sharq_quantize_weight(sharq_format fmt, const uint16_t *w_bf16, int64_t n, int64_t k,
                                   int64_t ld_w, const sharq_fp4_view *w_out, void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (!w_bf16 || !w_out || !w_out->codes) return SHARQ_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 || ld_w < k || w_out->ld_codes < k / 2) return SHARQ_ERR_SHAPE;
  if (ld_w % 8 || !aligned(w_bf16, 16) || !aligned(w_out->codes, 16) || w_out->ld_codes % 16)
    return SHARQ_ERR_ALIGN;
  sharq_status st = check_scales(fmt, w_out, n, k, false);
  if (st != SHARQ_OK) return st;
  if (fmt == SHARQ_NVFP4) {
    if (!w_out->tensor_scale) return SHARQ_ERR_NULL;
    if (!aligned(w_out->tensor_scale, 4)) return SHARQ_ERR_ALIGN;
  }
  QuantArgs a{w_bf16, ld_w, n, k, w_out->codes, w_out->ld_codes, w_out->scales, w_out->ld_scales,
              w_out->tensor_scale, kstep(w_out)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(fmt == SHARQ_MXFP4 ? sharq::launch_quantize_weight_mx(a, s)
                                     : sharq::launch_quantize_weight_nv(a, s));
}

sharq_status sharq_prepare(sharq_format fmt, const uint16_t *x_bf16, int64_t m, int64_t k,
                           int64_t ld_x, const uint16_t *gamma_bf16, float eps,
                           const sharq_fp4_view *sp, const sharq_fp4_view *rs, void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (!x_bf16 || !sp || !rs || !sp->codes || !sp->meta || !rs->codes) return SHARQ_ERR_NULL;
  if (m < 1 || k < 32 || k % 32 || ld_x < k) return SHARQ_ERR_SHAPE;
  if (gamma_bf16 && k > 16384) return SHARQ_ERR_UNSUPPORTED;
  if (sp->ld_codes < k / 4 || sp->ld_meta < k / 8 || rs->ld_codes < k / 2) return SHARQ_ERR_SHAPE;
  if (sp->dense_codes && sp->ld_dense < k / 2) return SHARQ_ERR_SHAPE;
  if (ld_x % 8 || !aligned(x_bf16, 16)) return SHARQ_ERR_ALIGN;
  if (gamma_bf16 && !aligned(gamma_bf16, 16)) return SHARQ_ERR_ALIGN;
  if (!aligned(sp->codes, 8) || sp->ld_codes % 8) return SHARQ_ERR_ALIGN;
  if (!aligned(sp->meta, 4) || sp->ld_meta % 4) return SHARQ_ERR_ALIGN;
  if (!aligned(rs->codes, 16) || rs->ld_codes % 16) return SHARQ_ERR_ALIGN;
  if (sp->dense_codes && (!aligned(sp->dense_codes, 16) || sp->ld_dense % 16)) return SHARQ_ERR_ALIGN;
  sharq_status st = check_scales(fmt, sp, m, k, false);
  if (st != SHARQ_OK) return st;
  st = check_scales(fmt, rs, m, k, false);
  if (st != SHARQ_OK) return st;
  if (fmt == SHARQ_NVFP4) {
    if (!sp->tensor_scale) return SHARQ_ERR_NULL;
    if (rs->tensor_scale && rs->tensor_scale != sp->tensor_scale) return SHARQ_ERR_SHAPE;
    if (!aligned(sp->tensor_scale, 4)) return SHARQ_ERR_ALIGN;
  }
  PrepArgs a{x_bf16, ld_x, m, k, gamma_bf16, eps,
             sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->scales, sp->ld_scales,
             rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             sp->dense_codes, sp->ld_dense, sp->tensor_scale, kstep(sp), kstep(rs)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(fmt == SHARQ_MXFP4 ? sharq::launch_prepare_mx(a, s)
                                     : sharq::launch_prepare_nv(a, s));
}

sharq_status sharq_dual_gemm(sharq_format fmt, const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                             const sharq_fp4_view *wsv, const sharq_fp4_view *wdv, int64_t m,
                             int64_t n, int64_t k, float *y, int64_t ld_y,
                             sharq_gemm_variant variant, void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (variant < SHARQ_GEMM_AUTO || variant > SHARQ_GEMM_SPARSE_MFMA) return SHARQ_ERR_UNSUPPORTED;
  if (!sp || !rs || !wsv || !wdv || !y) return SHARQ_ERR_NULL;
  if (!rs->codes || !wsv->codes || !wdv->codes) return SHARQ_ERR_NULL;
  if (m < 1 || n < 1 || k < 128 || k % 128 || ld_y < n) return SHARQ_ERR_SHAPE;
  // one weight payload, two scale views
  if (wsv->codes != wdv->codes || wsv->ld_codes != wdv->ld_codes) return SHARQ_ERR_SHAPE;
  if (fmt == SHARQ_MXFP4 && variant == SHARQ_GEMM_SPARSE_MFMA) return SHARQ_ERR_UNSUPPORTED;
  // AUTO reads the dense backbone view when the caller has one (no expansion
  // work in the GEMM), else the 2:4 form
  const bool dense_expanded = variant == SHARQ_GEMM_DENSE_EXPANDED ||
                              (variant == SHARQ_GEMM_AUTO && sp->dense_codes != nullptr);
  if (dense_expanded) {
    if (!sp->dense_codes) return SHARQ_ERR_NULL;
    if (sp->ld_dense < k / 2) return SHARQ_ERR_SHAPE;
    if (!aligned(sp->dense_codes, 16) || sp->ld_dense % 16) return SHARQ_ERR_ALIGN;
  } else {
    if (!sp->codes || !sp->meta) return SHARQ_ERR_NULL;
    if (sp->ld_codes < k / 4 || sp->ld_meta < k / 8) return SHARQ_ERR_SHAPE;
    if (!aligned(sp->codes, 16) || sp->ld_codes % 16 || !aligned(sp->meta, 8) || sp->ld_meta % 8)
      return SHARQ_ERR_ALIGN;
  }
  if (rs->ld_codes < k / 2 || wsv->ld_codes < k / 2) return SHARQ_ERR_SHAPE;
  if (!aligned(rs->codes, 16) || rs->ld_codes % 16 || !aligned(wsv->codes, 16) || wsv->ld_codes % 16)
    return SHARQ_ERR_ALIGN;
  if (!aligned(y, 4)) return SHARQ_ERR_ALIGN;
  sharq_status st;
  if ((st = check_scales(fmt, sp, m, k, true)) != SHARQ_OK) return st;
  if ((st = check_scales(fmt, rs, m, k, true)) != SHARQ_OK) return st;
  if ((st = check_scales(fmt, wsv, n, k, true)) != SHARQ_OK) return st;
  if ((st = check_scales(fmt, wdv, n, k, true)) != SHARQ_OK) return st;
  if (fmt == SHARQ_NVFP4) {
    if (!sp->tensor_scale || !wsv->tensor_scale) return SHARQ_ERR_NULL;
    if (!aligned(sp->tensor_scale, 4) || !aligned(wsv->tensor_scale, 4)) return SHARQ_ERR_ALIGN;
  }
  GemmArgs a{sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->dense_codes, sp->ld_dense,
             sp->scales, sp->ld_scales, rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             wsv->codes, wsv->ld_codes, wsv->scales, wsv->ld_scales, wdv->scales, wdv->ld_scales,
             sp->tensor_scale, wsv->tensor_scale, y, ld_y, m, n, k,
             kstep(sp), kstep(rs), kstep(wsv), kstep(wdv)};
  // the kernels address every operand with 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 32;
  if (m * rs->ld_codes >= lim || n * wsv->ld_codes >= lim ||
      (dense_expanded ? m * sp->ld_dense : m * sp->ld_codes) >= lim ||
      (!dense_expanded && m * sp->ld_meta >= lim) || !scales_fit(fmt, sp, m, k) ||
      !scales_fit(fmt, rs, m, k) || !scales_fit(fmt, wsv, n, k) || !scales_fit(fmt, wdv, n, k))
    return SHARQ_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == SHARQ_MXFP4) return from_hip(sharq::launch_dual_gemm_mx(a, dense_expanded, s));
  const int v = variant == SHARQ_GEMM_SPARSE_MFMA ? 3 : dense_expanded ? 2 : 1;
  return from_hip(sharq::launch_dual_gemm_nv(a, v, s));
}

}  // extern "C"
