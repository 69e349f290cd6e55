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

// A view's layout field: a known layout, reserved 0, k-step-major needs k % 128.
sharq_status check_layout(const sharq_fp4_view *v, int64_t k) {
  if (v->reserved != 0) return SHARQ_ERR_SHAPE;
  if (v->layout == SHARQ_LAYOUT_KSTEP_MAJOR) return k % 128 ? SHARQ_ERR_SHAPE : SHARQ_OK;
  return v->layout == SHARQ_LAYOUT_ROW_MAJOR ? SHARQ_OK : SHARQ_ERR_UNSUPPORTED;
}

// One array of a view with `rows` rows: `bpr` bytes per row (row-major), `bps`
// bytes per row and 128-k step (k-step-major); `rm_align` the row-major
// pointer and ld alignment, `ks_align` the k-step-major pointer alignment.
// Also bounds the array's extent: the kernels address it with 32-bit offsets.
sharq_status check_array(const void *p, int64_t ld, int layout, int64_t rows, int64_t k, int64_t bpr,
                         int rm_align, int64_t bps, int ks_align) {
  if (!p) return SHARQ_ERR_NULL;
  const int64_t lim = (int64_t)1 << 32;
  if (layout == SHARQ_LAYOUT_KSTEP_MAJOR) {
    if (ld < rows || (k / 128) * ld * bps >= lim) return SHARQ_ERR_SHAPE;
    if (!aligned(p, ks_align)) return SHARQ_ERR_ALIGN;
  } else {
    if (ld < bpr || rows * ld >= lim) return SHARQ_ERR_SHAPE;
    if (!aligned(p, rm_align) || ld % rm_align) return SHARQ_ERR_ALIGN;
  }
  return SHARQ_OK;
}

// Scale array of a view: GEMM reads whole 4-byte words; NVFP4 writers store 2 bytes.
sharq_status check_scales(sharq_format f, const sharq_fp4_view *v, int64_t rows, int64_t k, bool dword) {
  const int blk = block_of(f);
  const int rm_align = dword ? 4 : (f == SHARQ_NVFP4 ? 2 : 1);
  return check_array(v->scales, v->ld_scales, v->layout, rows, k, k / blk, rm_align, 128 / blk,
                     f == SHARQ_MXFP4 ? 4 : 8);
}

int ksm(const sharq_fp4_view *v) { return v->layout == SHARQ_LAYOUT_KSTEP_MAJOR ? 1 : 0; }

#define CHECK(expr)                          \
  do {                                       \
    const sharq_status st_ = (expr);         \
    if (st_ != SHARQ_OK) return st_;         \
  } while (0)

// The two views a preparation writes, for `rows` rows of length k: one layout,
// 2:4 codes, meta, residual codes, the optional dense backbone view and the
// scales as the writers store them.
sharq_status check_prep_views(sharq_format fmt, const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                              int64_t rows, int64_t k) {
  CHECK(check_layout(sp, k));
  CHECK(check_layout(rs, k));
  if (sp->layout != rs->layout) return SHARQ_ERR_SHAPE;
  const int L = sp->layout;
  CHECK(check_array(sp->codes, sp->ld_codes, L, rows, k, k / 4, 8, 32, 16));
  CHECK(check_array(sp->meta, sp->ld_meta, L, rows, k, k / 8, 4, 16, 16));
  CHECK(check_array(rs->codes, rs->ld_codes, L, rows, k, k / 2, 16, 64, 16));
  if (sp->dense_codes) CHECK(check_array(sp->dense_codes, sp->ld_dense, L, rows, k, k / 2, 16, 64, 16));
  CHECK(check_scales(fmt, sp, rows, k, false));
  CHECK(check_scales(fmt, rs, rows, k, false));
  return SHARQ_OK;
}

// The operands of the dense-view GEMM kernels (grouped and gate+up forms):
// `a_rows` activation rows with the dense backbone view, `w_rows` weight rows
// given as two views of one payload.
sharq_status check_dense_gemm_views(sharq_format fmt, const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                                    const sharq_fp4_view *wsv, const sharq_fp4_view *wdv, int64_t a_rows,
                                    int64_t w_rows, int64_t k) {
  CHECK(check_layout(sp, k));
  CHECK(check_layout(rs, k));
  CHECK(check_layout(wsv, k));
  CHECK(check_layout(wdv, k));
  if (!wsv->codes || !wdv->codes) return SHARQ_ERR_NULL;
  if (wsv->codes != wdv->codes || wsv->ld_codes != wdv->ld_codes || wsv->layout != wdv->layout)
    return SHARQ_ERR_SHAPE;
  if (!sp->dense_codes) return SHARQ_ERR_UNSUPPORTED;   // reads the dense backbone view
  CHECK(check_array(sp->dense_codes, sp->ld_dense, sp->layout, a_rows, k, k / 2, 16, 64, 16));
  CHECK(check_array(rs->codes, rs->ld_codes, rs->layout, a_rows, k, k / 2, 16, 64, 16));
  CHECK(check_array(wsv->codes, wsv->ld_codes, wsv->layout, w_rows, k, k / 2, 16, 64, 16));
  CHECK(check_scales(fmt, sp, a_rows, k, true));
  CHECK(check_scales(fmt, rs, a_rows, k, true));
  CHECK(check_scales(fmt, wsv, w_rows, k, true));
  CHECK(check_scales(fmt, wdv, w_rows, k, true));
  return SHARQ_OK;
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
  if (!w_bf16 || !w_out) return SHARQ_ERR_NULL;
  if (n < 1 || k < 32 || k % 32 || ld_w < k) return SHARQ_ERR_SHAPE;
  if (ld_w % 8 || !aligned(w_bf16, 16)) return SHARQ_ERR_ALIGN;
  CHECK(check_layout(w_out, k));
  CHECK(check_array(w_out->codes, w_out->ld_codes, w_out->layout, n, k, k / 2, 16, 64, 16));
  CHECK(check_scales(fmt, w_out, n, k, false));
  if (fmt == SHARQ_NVFP4) {
    if (!w_out->tensor_scale) return SHARQ_ERR_NULL;
    if (!aligned(w_out->tensor_scale, 4)) return SHARQ_ERR_ALIGN;
  }
  QuantArgs a{w_bf16, ld_w, n, k, w_out->codes, w_out->ld_codes, w_out->scales, w_out->ld_scales,
              w_out->tensor_scale, ksm(w_out)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(fmt == SHARQ_MXFP4 ? sharq::launch_quantize_weight_mx(a, s)
                                     : sharq::launch_quantize_weight_nv(a, s));
}

namespace {

// Row strides of the preparation's row inputs (bf16 X, h, o, x_out; fp32
// gate, up): the kernels address a group of up to 16 rows with 32-bit offsets
// from a per-group base (15 x 4 B x 2^26 < 2^32).
constexpr int64_t kMaxRowStride = (int64_t)1 << 26;

// Validation and launch shared by sharq_prepare and sharq_prepare_residual
// (add == nullptr: no residual add).
sharq_status prepare_common(sharq_format fmt, const uint16_t *x_bf16, int64_t m, int64_t k,
                            int64_t ld_x, const uint16_t *gamma_bf16, float eps,
                            const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                            const uint16_t *add, int64_t ld_add, uint16_t *x_out, int64_t ld_out,
                            void *stream, bool noalloc = false) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (!x_bf16 || !sp || !rs) return SHARQ_ERR_NULL;
  if (m < 1 || k < 32 || k % 32 || ld_x < k) return SHARQ_ERR_SHAPE;
  if (gamma_bf16 && k > 16384) return SHARQ_ERR_UNSUPPORTED;
  if (ld_x >= kMaxRowStride || (add && (ld_add >= kMaxRowStride || ld_out >= kMaxRowStride)))
    return SHARQ_ERR_UNSUPPORTED;
  if (ld_x % 8 || !aligned(x_bf16, 16)) return SHARQ_ERR_ALIGN;
  if (gamma_bf16 && !aligned(gamma_bf16, 16)) return SHARQ_ERR_ALIGN;
  CHECK(check_prep_views(fmt, sp, rs, m, k));
  if (fmt == SHARQ_NVFP4) {
    if (!sp->tensor_scale) return SHARQ_ERR_NULL;
    if (rs->tensor_scale && rs->tensor_scale != sp->tensor_scale) return SHARQ_ERR_SHAPE;
    if (!aligned(sp->tensor_scale, 4)) return SHARQ_ERR_ALIGN;
  }
  PrepArgs a{x_bf16, ld_x, m, k, gamma_bf16, eps,
             sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->scales, sp->ld_scales,
             rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             sp->dense_codes, sp->ld_dense, sp->tensor_scale, ksm(sp), ksm(rs)};
  a.add = add;
  a.ld_add = ld_add;
  a.x_out = x_out;
  a.ld_xout = ld_out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (noalloc) return from_hip(sharq::launch_prepare_noalloc(a, fmt == SHARQ_MXFP4 ? 0 : 1, s));
  a.amax = fmt == SHARQ_NVFP4 ? sp->tensor_scale + 1 : nullptr;
  return from_hip(fmt == SHARQ_MXFP4 ? sharq::launch_prepare_mx(a, s)
                                     : sharq::launch_prepare_nv(a, s));
}

}  // namespace

sharq_status sharq_prepare(sharq_format fmt, const uint16_t *x_bf16, int64_t m, int64_t k,
                           int64_t ld_x, const uint16_t *gamma_bf16, float eps,
                           const sharq_fp4_view *sp, const sharq_fp4_view *rs, void *stream) {
  return prepare_common(fmt, x_bf16, m, k, ld_x, gamma_bf16, eps, sp, rs, nullptr, 0, nullptr, 0,
                        stream);
}

sharq_status sharq_prepare_noalloc(sharq_format fmt, const uint16_t *x_bf16, int64_t m, int64_t k,
                                   int64_t ld_x, const uint16_t *gamma_bf16, float eps,
                                   const sharq_fp4_view *sp, const sharq_fp4_view *rs, void *stream) {
  return prepare_common(fmt, x_bf16, m, k, ld_x, gamma_bf16, eps, sp, rs, nullptr, 0, nullptr, 0,
                        stream, true);
}

sharq_status sharq_prepare_residual(sharq_format fmt, const uint16_t *h_bf16, int64_t ld_h,
                                    const uint16_t *o_bf16, int64_t ld_o, uint16_t *x_out_bf16,
                                    int64_t ld_out, int64_t m, int64_t k,
                                    const uint16_t *gamma_bf16, float eps,
                                    const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                                    void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (fmt != SHARQ_MXFP4) return SHARQ_ERR_UNSUPPORTED;
  if (!h_bf16 || !o_bf16 || !x_out_bf16 || !gamma_bf16) return SHARQ_ERR_NULL;
  if (ld_o < k || ld_out < k) return SHARQ_ERR_SHAPE;
  if (ld_o % 8 || ld_out % 8 || !aligned(o_bf16, 16) || !aligned(x_out_bf16, 16)) return SHARQ_ERR_ALIGN;
  // in place on h or o only with that array's own row stride
  if ((x_out_bf16 == h_bf16 && ld_out != ld_h) || (x_out_bf16 == o_bf16 && ld_out != ld_o))
    return SHARQ_ERR_SHAPE;
  return prepare_common(fmt, h_bf16, m, k, ld_h, gamma_bf16, eps, sp, rs, o_bf16, ld_o, x_out_bf16,
                        ld_out, stream);
}

sharq_status sharq_prepare_silu_mul(sharq_format fmt, const float *gate, int64_t ld_gate,
                                    const float *up, int64_t ld_up, int64_t m, int64_t k,
                                    const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                                    void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (fmt != SHARQ_MXFP4) return SHARQ_ERR_UNSUPPORTED;
  if (!gate || !up || !sp || !rs) return SHARQ_ERR_NULL;
  if (m < 1 || k < 32 || k % 32 || ld_gate < k || ld_up < k) return SHARQ_ERR_SHAPE;
  if (ld_gate >= kMaxRowStride || ld_up >= kMaxRowStride) return SHARQ_ERR_UNSUPPORTED;
  if (ld_gate % 4 || ld_up % 4 || !aligned(gate, 16) || !aligned(up, 16)) return SHARQ_ERR_ALIGN;
  CHECK(check_prep_views(fmt, sp, rs, m, k));
  PrepArgs a{nullptr, 0, m, k, nullptr, 0.0f,
             sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->scales, sp->ld_scales,
             rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             sp->dense_codes, sp->ld_dense, nullptr, ksm(sp), ksm(rs)};
  a.gate = gate;
  a.ld_gate = ld_gate;
  a.up = up;
  a.ld_up = ld_up;
  return from_hip(sharq::launch_prepare_silu_mx(a, static_cast<hipStream_t>(stream)));
}

sharq_status sharq_dual_gemm_silu_prepare(sharq_format fmt, const sharq_fp4_view *sp,
                                          const sharq_fp4_view *rs, const sharq_fp4_view *wsv,
                                          const sharq_fp4_view *wdv, int64_t m, int64_t inter,
                                          int64_t k, const sharq_fp4_view *sp_out,
                                          const sharq_fp4_view *rs_out, void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (fmt != SHARQ_MXFP4) return SHARQ_ERR_UNSUPPORTED;
  if (!sp || !rs || !wsv || !wdv || !sp_out || !rs_out) return SHARQ_ERR_NULL;
  if (m < 1 || inter < 128 || inter % 128 || k < 128 || k % 128) return SHARQ_ERR_SHAPE;
  const int64_t n = 2 * inter;
  CHECK(check_dense_gemm_views(fmt, sp, rs, wsv, wdv, m, n, k));
  CHECK(check_prep_views(fmt, sp_out, rs_out, m, inter));   // the preparation of x [m, inter]
  GemmArgs a{sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->dense_codes, sp->ld_dense,
             sp->scales, sp->ld_scales, rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             wsv->codes, wsv->ld_codes, wsv->scales, wsv->ld_scales, wdv->scales, wdv->ld_scales,
             nullptr, nullptr, nullptr, 0, m, n, k, ksm(sp), ksm(rs), ksm(wsv)};
  PrepArgs o{nullptr, 0, m, inter, nullptr, 0.0f,
             sp_out->codes, sp_out->ld_codes, sp_out->meta, sp_out->ld_meta, sp_out->scales,
             sp_out->ld_scales, rs_out->codes, rs_out->ld_codes, rs_out->scales, rs_out->ld_scales,
             sp_out->dense_codes, sp_out->ld_dense, nullptr, ksm(sp_out), ksm(rs_out)};
  return from_hip(sharq::launch_dual_gemm_silu_prep_mx(a, o, static_cast<hipStream_t>(stream)));
}

sharq_status sharq_grouped_dual_gemm_silu_prepare(
    sharq_format fmt, const sharq_fp4_view *sp, const sharq_fp4_view *rs, int64_t tokens,
    const int32_t *row_index, const int64_t *group_offsets, int64_t groups, int64_t rows,
    const sharq_fp4_view *wsv, const sharq_fp4_view *wdv, int64_t inter, int64_t k,
    const sharq_fp4_view *sp_out, const sharq_fp4_view *rs_out, void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (fmt != SHARQ_MXFP4) return SHARQ_ERR_UNSUPPORTED;
  if (!sp || !rs || !wsv || !wdv || !group_offsets || !sp_out || !rs_out) return SHARQ_ERR_NULL;
  if (groups < 1 || groups > 256) return SHARQ_ERR_UNSUPPORTED;
  if (tokens < 1 || rows < 0 || inter < 128 || inter % 128 || k < 128 || k % 128) return SHARQ_ERR_SHAPE;
  if (!row_index && rows > tokens) return SHARQ_ERR_SHAPE;
  if (!aligned(group_offsets, 8) || (row_index && !aligned(row_index, 4))) return SHARQ_ERR_ALIGN;
  const int64_t n = 2 * inter;
  CHECK(check_dense_gemm_views(fmt, sp, rs, wsv, wdv, tokens, groups * n, k));
  CHECK(check_prep_views(fmt, sp_out, rs_out, rows > 0 ? rows : 1, inter));   // x [rows, inter]
  if (rows == 0) return SHARQ_OK;
  GemmArgs a{sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->dense_codes, sp->ld_dense,
             sp->scales, sp->ld_scales, rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             wsv->codes, wsv->ld_codes, wsv->scales, wsv->ld_scales, wdv->scales, wdv->ld_scales,
             nullptr, nullptr, nullptr, 0, rows, n, k, ksm(sp), ksm(rs), ksm(wsv)};
  a.row_index = row_index;
  a.group_off = group_offsets;
  a.groups = groups;
  a.tokens = tokens;
  PrepArgs o{nullptr, 0, rows, inter, nullptr, 0.0f,
             sp_out->codes, sp_out->ld_codes, sp_out->meta, sp_out->ld_meta, sp_out->scales,
             sp_out->ld_scales, rs_out->codes, rs_out->ld_codes, rs_out->scales, rs_out->ld_scales,
             sp_out->dense_codes, sp_out->ld_dense, nullptr, ksm(sp_out), ksm(rs_out)};
  return from_hip(sharq::launch_grouped_dual_gemm_silu_prep_mx(a, o, static_cast<hipStream_t>(stream)));
}

sharq_status sharq_grouped_dual_gemm(sharq_format fmt, const sharq_fp4_view *sp,
                                     const sharq_fp4_view *rs, int64_t tokens,
                                     const int32_t *row_index, const int64_t *group_offsets,
                                     int64_t groups, int64_t rows, const sharq_fp4_view *wsv,
                                     const sharq_fp4_view *wdv, int64_t n, int64_t k, float *y,
                                     int64_t ld_y, void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (fmt != SHARQ_MXFP4) return SHARQ_ERR_UNSUPPORTED;
  if (!sp || !rs || !wsv || !wdv || !y || !group_offsets) return SHARQ_ERR_NULL;
  if (groups < 1 || groups > 256) return SHARQ_ERR_UNSUPPORTED;
  if (tokens < 1 || rows < 0 || n < 1 || k < 128 || k % 128 || ld_y < n) return SHARQ_ERR_SHAPE;
  if (!row_index && rows > tokens) return SHARQ_ERR_SHAPE;
  if (!aligned(group_offsets, 8) || (row_index && !aligned(row_index, 4)) || !aligned(y, 4))
    return SHARQ_ERR_ALIGN;
  CHECK(check_dense_gemm_views(fmt, sp, rs, wsv, wdv, tokens, groups * n, k));
  if (rows == 0) return SHARQ_OK;
  GemmArgs a{sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->dense_codes, sp->ld_dense,
             sp->scales, sp->ld_scales, rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             wsv->codes, wsv->ld_codes, wsv->scales, wsv->ld_scales, wdv->scales, wdv->ld_scales,
             nullptr, nullptr, y, ld_y, rows, n, k, ksm(sp), ksm(rs), ksm(wsv)};
  a.row_index = row_index;
  a.group_off = group_offsets;
  a.groups = groups;
  a.tokens = tokens;
  return from_hip(sharq::launch_grouped_dual_gemm_mx(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Validation and launch shared by sharq_dual_gemm (fp32 Y) and
// sharq_dual_gemm_bf16 (y16: bf16 Y); exactly one of y and y16 is set.
sharq_status dual_gemm_common(sharq_format fmt, const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                              const sharq_fp4_view *wsv, const sharq_fp4_view *wdv, int64_t m,
                              int64_t n, int64_t k, float *y, uint16_t *y16, int64_t ld_y,
                              sharq_gemm_variant variant, void *stream) {
  if (!valid_format(fmt)) return SHARQ_ERR_UNSUPPORTED;
  if (variant < SHARQ_GEMM_AUTO || variant > SHARQ_GEMM_SPARSE_MFMA) return SHARQ_ERR_UNSUPPORTED;
  if (!sp || !rs || !wsv || !wdv || (!y && !y16)) return SHARQ_ERR_NULL;
  if (m < 1 || n < 1 || k < 128 || k % 128 || ld_y < n) return SHARQ_ERR_SHAPE;
  CHECK(check_layout(sp, k));
  CHECK(check_layout(rs, k));
  CHECK(check_layout(wsv, k));
  CHECK(check_layout(wdv, k));
  // one weight payload, two scale views
  if (!wsv->codes || !wdv->codes) return SHARQ_ERR_NULL;
  if (wsv->codes != wdv->codes || wsv->ld_codes != wdv->ld_codes || wsv->layout != wdv->layout)
    return SHARQ_ERR_SHAPE;
  // AUTO: NVFP4 runs the 2:4 backbone on the structured-sparse MFMA (its
  // fastest variant); MXFP4 reads the dense backbone view when the caller has
  // one (no expansion work in the GEMM), else the 2:4 form
  if (fmt == SHARQ_NVFP4 && variant == SHARQ_GEMM_AUTO) variant = SHARQ_GEMM_SPARSE_MFMA;
  const bool dense_expanded = variant == SHARQ_GEMM_DENSE_EXPANDED ||
                              (variant == SHARQ_GEMM_AUTO && sp->dense_codes != nullptr);
  if (dense_expanded) {
    CHECK(check_array(sp->dense_codes, sp->ld_dense, sp->layout, m, k, k / 2, 16, 64, 16));
  } else {
    CHECK(check_array(sp->codes, sp->ld_codes, sp->layout, m, k, k / 4, 16, 32, 16));
    CHECK(check_array(sp->meta, sp->ld_meta, sp->layout, m, k, k / 8, 8, 16, 16));
  }
  CHECK(check_array(rs->codes, rs->ld_codes, rs->layout, m, k, k / 2, 16, 64, 16));
  CHECK(check_array(wsv->codes, wsv->ld_codes, wsv->layout, n, k, k / 2, 16, 64, 16));
  if (y ? !aligned(y, 4) : !aligned(y16, 2)) return SHARQ_ERR_ALIGN;
  CHECK(check_scales(fmt, sp, m, k, true));
  CHECK(check_scales(fmt, rs, m, k, true));
  CHECK(check_scales(fmt, wsv, n, k, true));
  CHECK(check_scales(fmt, wdv, n, k, true));
  if (fmt == SHARQ_NVFP4) {
    if (!sp->tensor_scale || !wsv->tensor_scale) return SHARQ_ERR_NULL;
    if (!aligned(sp->tensor_scale, 4) || !aligned(wsv->tensor_scale, 4)) return SHARQ_ERR_ALIGN;
  }
  GemmArgs a{sp->codes, sp->ld_codes, sp->meta, sp->ld_meta, sp->dense_codes, sp->ld_dense,
             sp->scales, sp->ld_scales, rs->codes, rs->ld_codes, rs->scales, rs->ld_scales,
             wsv->codes, wsv->ld_codes, wsv->scales, wsv->ld_scales, wdv->scales, wdv->ld_scales,
             sp->tensor_scale, wsv->tensor_scale, y, ld_y, m, n, k,
             ksm(sp), ksm(rs), ksm(wsv)};
  a.y16 = y16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == SHARQ_MXFP4 && variant == SHARQ_GEMM_SPARSE_MFMA) return from_hip(sharq::launch_dual_gemm_mx_fp8sp(a, s));
  if (fmt == SHARQ_MXFP4) return from_hip(sharq::launch_dual_gemm_mx(a, dense_expanded, s));
  const int v = variant == SHARQ_GEMM_SPARSE_MFMA ? 3 : dense_expanded ? 2 : 1;
  return from_hip(sharq::launch_dual_gemm_nv(a, v, s));
}

}  // namespace

extern "C" {

sharq_status sharq_dual_gemm(sharq_format fmt, const sharq_fp4_view *sp, const sharq_fp4_view *rs,
                             const sharq_fp4_view *wsv, const sharq_fp4_view *wdv, int64_t m,
                             int64_t n, int64_t k, float *y, int64_t ld_y,
                             sharq_gemm_variant variant, void *stream) {
  if (!y) return SHARQ_ERR_NULL;
  return dual_gemm_common(fmt, sp, rs, wsv, wdv, m, n, k, y, nullptr, ld_y, variant, stream);
}

sharq_status sharq_dual_gemm_bf16(sharq_format fmt, const sharq_fp4_view *sp,
                                  const sharq_fp4_view *rs, const sharq_fp4_view *wsv,
                                  const sharq_fp4_view *wdv, int64_t m, int64_t n, int64_t k,
                                  uint16_t *y_bf16, int64_t ld_y, sharq_gemm_variant variant,
                                  void *stream) {
  if (!y_bf16) return SHARQ_ERR_NULL;
  return dual_gemm_common(fmt, sp, rs, wsv, wdv, m, n, k, nullptr, y_bf16, ld_y, variant, stream);
}

}  // extern "C"
