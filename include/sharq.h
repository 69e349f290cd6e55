/*
 * sharq.h - C ABI of the SharQ linear-layer hot path for AMD Instinct MI355X (gfx950).
 *
 * The operations follow "SharQ: Bridging Activation Sparsity and FP4
 * Quantization for LLM Inference" (arXiv:2606.26587), abstract:
 *   - sentence 3: per activation tensor, an input-adaptive N:M mask extracts an
 *     outlier-dominated sparse backbone that is quantized to FP4, and a dense
 *     residual is formed against the QUANTIZED backbone;
 *   - sentence 4: a sparse-path FP4 GEMM on the backbone plus a dense-path FP4
 *     GEMM on the residual;
 *   - sentence 5: both paths read one FP4 weight payload through path-specific
 *     scale views; one fused preparation operator does the layer
 *     normalization, mask generation and residual construction;
 *   - sentence 7: MXFP4 and NVFP4 formats.
 * Concrete readings (2:4 along K, RMSNorm, block sizes, rounding) are stated
 * at each entry point.  Beyond the path itself, sharq_prepare_residual and
 * sharq_prepare_silu_mul fuse the decoder layer's neighbouring steps (the
 * residual add, SiLU(gate) * up) into the preparation,
 * sharq_dual_gemm_silu_prepare runs the gate+up GEMM with SiLU(gate) * up and
 * the down projection's preparation in its epilogue, and
 * sharq_grouped_dual_gemm (and its _silu_prepare form) runs a
 * mixture-of-experts layer's expert GEMMs.
 *
 * Conventions for every entry point:
 *   - All matrices are row-major, K contiguous.  X is [m, k] bf16, W is
 *     [n, k] bf16, Y = X * W^T is [m, n] fp32.  bf16 values are passed as
 *     their uint16 bit patterns.
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     allocates nothing, keeps no state between calls and never synchronizes
 *     (sharq_prepare_noalloc alone keeps a 256-byte static workspace per GPU).
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and is complete when the stream is.
 *   - Leading dimensions (`ld_*`) are in elements of the array they describe
 *     (bytes for uint8 arrays).
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is enqueued.  A launch failure reported by the HIP runtime
 *     returns SHARQ_ERR_DEVICE; faults inside kernels surface at the caller's
 *     next synchronization.  No C++ exception crosses this interface.
 *   - Inputs must be finite (no NaN or Inf).
 *   - Calls on different streams that write the same buffers race.
 */
#ifndef SHARQ_H
#define SHARQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SHARQ_OK = 0,
    SHARQ_ERR_NULL = 1,        /* a required pointer is NULL */
    SHARQ_ERR_SHAPE = 2,       /* a size, leading dimension or view pairing is invalid */
    SHARQ_ERR_ALIGN = 3,       /* a pointer or leading dimension is misaligned */
    SHARQ_ERR_UNSUPPORTED = 4, /* valid request this build or the ISA cannot serve */
    SHARQ_ERR_DEVICE = 5       /* the HIP runtime reported an error at launch */
} sharq_status;

typedef enum {
    /* E2M1 elements, one E8M0 scale (2^(byte-127)) per 32 consecutive k (OCP MX v1.0) */
    SHARQ_MXFP4 = 0,
    /* E2M1 elements, one E4M3 scale per 16 consecutive k, and one fp32 tensor scale */
    SHARQ_NVFP4 = 1
} sharq_format;

typedef enum {
    SHARQ_GEMM_AUTO = 0,           /* the format's default (see sharq_dual_gemm) */
    SHARQ_GEMM_DECOMPRESS = 1,     /* backbone expanded from its 2:4 form to dense FP4 while staged in LDS */
    SHARQ_GEMM_DENSE_EXPANDED = 2, /* backbone read from the dense view written by sharq_prepare */
    SHARQ_GEMM_SPARSE_MFMA = 3     /* backbone on a structured-sparse MFMA (see sharq_dual_gemm) */
} sharq_gemm_variant;

/*
 * Layout of every array of one operand view (sharq_fp4_view.layout): codes,
 * meta, dense_codes and scales alike.
 *   ROW_MAJOR:   row r of an array starts at array + r * ld (ld in bytes) and
 *                holds the row's bytes in k order (see sharq_fp4_view).
 *   KSTEP_MAJOR: k is cut into steps of 128; the bytes of row r that belong to
 *                step t are contiguous, and so are the rows of one step: they
 *                start at array + (t * ld + r) * b, where b is the array's bytes
 *                per row and step (dense codes 64, 2:4 codes 32, meta 16, scales
 *                4 for MXFP4 and 8 for NVFP4) and ld >= rows counts rows per
 *                step.  Needs k % 128 == 0.  This is the layout the GEMM
 *                streams fastest: 16 rows of one step are 1 KiB of contiguous
 *                codes, so every cache line it fetches is used whole.
 */
typedef enum {
    SHARQ_LAYOUT_ROW_MAJOR = 0,
    SHARQ_LAYOUT_KSTEP_MAJOR = 1
} sharq_layout;

/* Which array sharq_bytes sizes. */
enum {
    SHARQ_BYTES_DENSE_CODES = 0,   /* dense FP4 codes: rows x k/2 */
    SHARQ_BYTES_SPARSE_CODES = 1,  /* 2:4-compressed backbone codes: rows x k/4 */
    SHARQ_BYTES_META = 2,          /* 2:4 indices: rows x k/8 */
    SHARQ_BYTES_SCALES = 3         /* block scales: rows x k/32 (MX) or k/16 (NV) */
};

/*
 * One FP4 operand view; all pointers are device pointers, every array in the
 * layout `layout` names.  Per row, in k order:
 *
 *   codes        dense operand: k/2 bytes, two E2M1 codes per byte, the lower
 *                k in the low nibble.  2:4 backbone: k/4 bytes, one byte per
 *                group of four k: the code of the lower kept index in the low
 *                nibble, the code of the higher kept index in the high nibble.
 *   meta         backbone only (else NULL): k/8 bytes; per group of four k the
 *                nibble i0 | i1 << 2 (kept indices, i0 < i1); group 2j sits in
 *                the low nibble of byte j.
 *   scales       E8M0 bytes (MXFP4, one per 32 k) or E4M3 bytes (NVFP4, one per
 *                16 k).
 *   dense_codes  optional backbone in the dense layout of `codes` (zeros at the
 *                dropped positions); written by sharq_prepare when non-NULL and
 *                read by SHARQ_GEMM_DENSE_EXPANDED.  NULL otherwise.
 *   tensor_scale NVFP4: device float[2]; [0] is the fp32 tensor scale, [1] is
 *                the amax the library reduces into while computing it.  MXFP4: NULL.
 */
typedef struct sharq_fp4_view {
    uint8_t *codes;
    int64_t ld_codes;
    uint8_t *meta;
    int64_t ld_meta;
    uint8_t *scales;
    int64_t ld_scales;
    int32_t layout;         /* sharq_layout, for every array of the view */
    int32_t reserved;       /* must be 0 */
    uint8_t *dense_codes;
    int64_t ld_dense;
    float *tensor_scale;
} sharq_fp4_view;

/*
 * Requirements on a view of `rows` rows (checked by every entry point,
 * SHARQ_ERR_SHAPE / SHARQ_ERR_ALIGN otherwise):
 *   ROW_MAJOR:   each ld at least the array's row length in bytes (codes k/2,
 *                or k/4 for 2:4 codes, meta k/8, dense_codes k/2, scales k/32
 *                for MXFP4 and k/16 for NVFP4); codes and dense_codes 16-byte
 *                aligned with ld % 16 == 0 (2:4 codes written by sharq_prepare:
 *                8 and 8; read by the GEMM: 16 and 16); meta 4-byte aligned
 *                with ld % 4 == 0 (read by the GEMM: 8 and 8); scales 4-byte
 *                aligned with ld % 4 == 0 for the GEMM, 2-byte and even for
 *                NVFP4 writers.
 *   KSTEP_MAJOR: k % 128 == 0; each ld >= rows; codes, meta and dense_codes
 *                16-byte aligned; scales 4-byte (MXFP4) or 8-byte (NVFP4)
 *                aligned.
 *   reserved == 0.
 */

/*
 * Quantize a weight matrix W [n, k] (bf16, row stride ld_w) to one FP4
 * payload (abstract, sentence 5: a single FP4 weight payload serves both
 * GEMM paths).  Each row is split into blocks of 32 (MX) or 16 (NV) along k:
 *   MXFP4: scale exponent e = floor(log2(amax)) - 2 clamped to [-127, 127]
 *          (e = -127 when amax = 0), byte e + 127; codes are E2M1 of w * 2^-e,
 *          round to nearest, ties to even, saturating at 6; the sign of zero
 *          is kept.
 *   NVFP4: tensor scale s_t = amax(W) / 2688 (1 when W is all zero), block
 *          scale byte = E4M3(amax_block / (6 s_t)) (nearest even, saturating
 *          at 448), S = e4m3(byte) * s_t, codes = E2M1(w / S); every step is
 *          one fp32 operation.
 * Writes w_out->codes (dense, n rows), w_out->scales, and for NVFP4
 * w_out->tensor_scale[0..1], in the layout w_out->layout names.  meta and
 * dense_codes are ignored.
 * Requirements: n >= 1, k >= 32, k % 32 == 0, ld_w >= k, ld_w % 8 == 0;
 * w_bf16 16-byte aligned; w_out as the view requirements above state.
 */
sharq_status sharq_quantize_weight(sharq_format fmt, const uint16_t *w_bf16, int64_t n,
                                   int64_t k, int64_t ld_w, const sharq_fp4_view *w_out,
                                   void *stream);

/*
 * The fused preparation operator (abstract, sentences 3 and 5), one HBM pass
 * over X [m, k] (bf16, row stride ld_x):
 *   1. RMSNorm when gamma_bf16 != NULL: ss = sum of x^2 as a perfect binary
 *      tree of fp32 additions over 2^ceil(log2 k) leaves (missing leaves 0,
 *      adjacent pairs); r = 1 / sqrt(ss / k + eps) with IEEE division and
 *      square root; x_n = bf16((x * r) * gamma).  gamma_bf16 == NULL: x_n = x.
 *   2. 2:4 mask: in every aligned group of four k keep the two largest |x_n|,
 *      the lower index first on ties.
 *   3. Backbone = x_n at kept positions, +0 elsewhere, quantized per block
 *      exactly as sharq_quantize_weight quantizes a weight row (NVFP4: with
 *      the activation tensor scale s_t = amax(x_n) / 2688, computed on the
 *      device by a reduction pass before the preparation pass).
 *   4. Residual R = x_n - deq(backbone) in fp32 (exact), quantized the same way
 *      (NVFP4: same s_t).
 * Outputs: sparse_out->codes (2:4-compressed), ->meta, ->scales and, when
 * non-NULL, ->dense_codes; resid_out->codes (dense) and ->scales; NVFP4:
 * sparse_out->tensor_scale[0..1] (resid_out->tensor_scale must be NULL or the
 * same pointer: one tensor scale serves both paths).
 * Requirements: m >= 1; k >= 32, k % 32 == 0; k <= 16384 when gamma is given;
 * ld_x >= k, ld_x % 8 == 0; x 16-byte aligned; both views as the view
 * requirements above state (m rows), with the same layout.  ld_x < 2^26
 * (SHARQ_ERR_UNSUPPORTED otherwise: the kernels address a group of rows of X
 * with 32-bit offsets from a per-group base).
 */
sharq_status sharq_prepare(sharq_format fmt, const uint16_t *x_bf16, int64_t m, int64_t k,
                           int64_t ld_x, const uint16_t *gamma_bf16, float eps,
                           const sharq_fp4_view *sparse_out, const sharq_fp4_view *resid_out,
                           void *stream);

/*
 * sharq_prepare for callers that cannot allocate, or whose calls must not
 * write beyond their outputs: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same operation, arguments, outputs
 * and requirements as sharq_prepare, with one difference: for NVFP4 the
 * tensor amax is reduced in a workspace the library holds in a file-scope
 * static device array (256 bytes on each GPU the library runs on, held until
 * the process ends) instead of in sparse_out->tensor_scale[1], so the caller's
 * tensor_scale needs one float ([0] receives s_t; [1] is not touched).  The
 * workspace holds one value whatever the shapes, so no size is refused for
 * it.  Nothing is allocated: no hipMalloc, hipFree or allocating library
 * call; the first call on a device takes the workspace's address there
 * (hipGetSymbolAddress) and keeps it.  Each call clears the workspace with a
 * kernel before using it.  Every call on one GPU shares the workspace, so
 * calls that overlap on one GPU (on different streams) race.  MXFP4 uses no
 * workspace: the call is exactly sharq_prepare's.
 */
sharq_status sharq_prepare_noalloc(sharq_format fmt, const uint16_t *x_bf16, int64_t m, int64_t k,
                                   int64_t ld_x, const uint16_t *gamma_bf16, float eps,
                                   const sharq_fp4_view *sparse_out,
                                   const sharq_fp4_view *resid_out, void *stream);

/*
 * The preparation operator with the residual add in front of its norm fused
 * in (the step the pre-norm decoder layer runs right before the norm that
 * the abstract, sentence 5, has the preparation absorb):
 *   x = bf16(h + o)   elementwise: the bf16 residual stream h [m, k] (row
 *                     stride ld_h) plus the bf16 sublayer output o (ld_o),
 *                     added in fp32 and rounded to nearest even;
 * x is stored to x_out (bf16, ld_out) as the new residual stream, and
 * sharq_prepare's steps 1-4 follow on x with gamma_bf16 (required) and eps.
 * One HBM pass over h and o.  x_out may be h itself (with ld_out == ld_h) or
 * o (with ld_out == ld_o); any other overlap is undefined.
 * MXFP4 only (SHARQ_ERR_UNSUPPORTED for NVFP4, whose tensor-scale pre-pass
 * would need the sum first).
 * Requirements: as sharq_prepare with gamma given, and for h, o and x_out:
 * ld >= k, ld % 8 == 0, ld < 2^26, 16-byte aligned.
 */
sharq_status sharq_prepare_residual(sharq_format fmt, const uint16_t *h_bf16, int64_t ld_h,
                                    const uint16_t *o_bf16, int64_t ld_o, uint16_t *x_out_bf16,
                                    int64_t ld_out, int64_t m, int64_t k,
                                    const uint16_t *gamma_bf16, float eps,
                                    const sharq_fp4_view *sparse_out,
                                    const sharq_fp4_view *resid_out, void *stream);

/*
 * The preparation operator with SiLU(gate) * up in front of it (the down
 * projection's input in a gated MLP; no norm):
 *   x = bf16(g / (1 + exp(-g)) * u)   elementwise over the fp32 gate g and up
 *                                     u [m, k] (row strides ld_gate, ld_up;
 *                                     e.g. the two halves of the gate+up
 *                                     projection's fp32 output), evaluated in
 *                                     binary64 and rounded once to nearest
 *                                     even (the kernel evaluates in fp32 and
 *                                     repeats in binary64 wherever fp32 could
 *                                     round differently);
 * then sharq_prepare's steps 2-4 on x (no normalization).  x itself is not
 * written.  One HBM pass over g and u.  MXFP4 only.
 * Requirements: m >= 1; k >= 32, k % 32 == 0; ld_gate, ld_up >= k,
 * multiples of 4 and below 2^26 (SHARQ_ERR_UNSUPPORTED otherwise); gate and
 * up 16-byte aligned; both views as sharq_prepare requires.  Inputs are
 * finite with |x| below the bf16 maximum.
 */
sharq_status sharq_prepare_silu_mul(sharq_format fmt, const float *gate, int64_t ld_gate,
                                    const float *up, int64_t ld_up, int64_t m, int64_t k,
                                    const sharq_fp4_view *sparse_out,
                                    const sharq_fp4_view *resid_out, void *stream);

/*
 * The gate+up projection of a gated MLP with the down projection's
 * preparation fused into its epilogue (the steps on either side of the path in
 * a decoder layer; abstract, sentences 3-5 for the GEMM and the preparation):
 *   Y = sharq_dual_gemm's product of (sparse, resid) [m, k] and the weight
 *       views [2 inter, k]: rows 0 .. inter - 1 of W are the gate projection,
 *       rows inter .. 2 inter - 1 the up projection;
 *   x = bf16(g / (1 + exp(-g)) * u) with g = Y[:, j], u = Y[:, inter + j]
 *       (the fp32 values sharq_dual_gemm would store), exactly as
 *       sharq_prepare_silu_mul forms it;
 *   then sharq_prepare's steps 2-4 on x [m, inter] (no normalization) into
 *   sparse_out and resid_out (dense_codes written when non-NULL).
 * Neither Y nor x is written: each workgroup forms x for 128 rows and 128
 * columns in LDS and prepares it there.  The outputs equal, byte for byte,
 * sharq_dual_gemm (MXFP4, DENSE_EXPANDED) followed by sharq_prepare_silu_mul
 * on the two halves of Y.
 * MXFP4 only; reads the dense backbone view (sparse->dense_codes required,
 * SHARQ_ERR_UNSUPPORTED otherwise).  The outputs must not overlap the inputs.
 * Built for prefill: it runs 128-row tiles, so for m <= 32 (decode) the
 * two-step path (sharq_dual_gemm, then sharq_prepare_silu_mul) is faster.
 * Requirements: m >= 1; inter >= 128, inter % 128 == 0; k >= 128,
 * k % 128 == 0; the input views as sharq_dual_gemm requires (m activation
 * rows, 2 inter weight rows, one payload); the output views as
 * sharq_prepare requires for m rows of length inter, with one layout.
 */
sharq_status sharq_dual_gemm_silu_prepare(sharq_format fmt, const sharq_fp4_view *sparse,
                                          const sharq_fp4_view *resid,
                                          const sharq_fp4_view *w_sparse_view,
                                          const sharq_fp4_view *w_dense_view, int64_t m,
                                          int64_t inter, int64_t k,
                                          const sharq_fp4_view *sparse_out,
                                          const sharq_fp4_view *resid_out, void *stream);

/*
 * Dual-path GEMM (abstract, sentences 4 and 5):
 *   Y = deq(backbone) * deq(W)^T + deq(residual) * deq(W)^T
 * accumulated in fp32 and stored as fp32 [m, n] (row stride ld_y).  NVFP4:
 * block values are exact (E2M1 x E4M3) and the two tensor scales are applied
 * to the fp32 sum.
 * The weight is passed as two views of ONE payload: w_sparse_view->codes must
 * equal w_dense_view->codes (otherwise SHARQ_ERR_SHAPE); each view brings its
 * own scales pointer (the path-specific scale view: the backbone product
 * reads w_sparse_view->scales, the residual product w_dense_view->scales;
 * usually both alias the weight's scales).  Both weight views must name the
 * same layout.
 * Variants: DECOMPRESS reads the 2:4 backbone (codes + meta) and expands it
 * to dense codes inside the GEMM; DENSE_EXPANDED reads sparse->dense_codes
 * instead; AUTO is, for MXFP4, DENSE_EXPANDED when sparse->dense_codes is
 * non-NULL, else DECOMPRESS, and for NVFP4 SPARSE_MFMA.  SPARSE_MFMA feeds
 * the 2:4 backbone codes and indices to a structured-sparse MFMA: for NVFP4
 * the fp16 one; for MXFP4, since gfx950 has no structured-sparse MFMA for FP4
 * operands, the FP8 one, after rebasing each backbone row and each weight
 * row (its w_sparse_view scales) to one power of two per row, which is exact
 * in E4M3 when the row's block scales span at most 12 binades; a 128 x 128
 * output tile with a row spanning more runs its backbone expanded to dense
 * FP4 instead.  The backbone product is then summed in its own fp32
 * accumulator and scaled by the two rows' powers of two.  The 2:4 indices
 * must be as sharq_prepare writes them (the two kept positions of a group
 * distinct).
 * NVFP4 runs on fp16 MFMAs (2:4 and dense): each operand element
 * q * e4m3 scale is exact in fp16.
 * Requirements: m, n >= 1; k >= 128, k % 128 == 0; ld_y >= n; y 4-byte
 * aligned; the four views as the view requirements above state (m rows for
 * the activations, n for the weight); every array spans less than 4 GiB.
 * Fastest when every view is KSTEP_MAJOR.
 */
sharq_status sharq_dual_gemm(sharq_format fmt, const sharq_fp4_view *sparse,
                             const sharq_fp4_view *resid, const sharq_fp4_view *w_sparse_view,
                             const sharq_fp4_view *w_dense_view, int64_t m, int64_t n, int64_t k,
                             float *y, int64_t ld_y, sharq_gemm_variant variant, void *stream);

/*
 * sharq_dual_gemm with a bf16 output (abstract, sentences 4 and 5: the same
 * dual-path product; the bf16 store is the epilogue a decoder layer's next
 * step reads, e.g. attention after QKV or the residual add after O and
 * down).  Y is accumulated in fp32 exactly as sharq_dual_gemm accumulates it
 * (same kernels, same summation order, same variants and AUTO choice) and
 * each value is rounded once to bf16, to nearest with ties to even, and
 * stored as its bit pattern into y_bf16 [m, n] (row stride ld_y elements).
 * So y_bf16 equals, bit for bit, the bf16 rounding of what sharq_dual_gemm
 * writes for the same inputs.  The rounding adds up to 2^-8 of |Y| per
 * value, more than the 1e-3 normwise budget of the fp32 output: use
 * sharq_dual_gemm where that budget matters.
 * Requirements: those of sharq_dual_gemm, with y_bf16 2-byte aligned.
 * Errors as sharq_dual_gemm (y_bf16 NULL: SHARQ_ERR_NULL).
 */
sharq_status sharq_dual_gemm_bf16(sharq_format fmt, const sharq_fp4_view *sparse,
                                  const sharq_fp4_view *resid, const sharq_fp4_view *w_sparse_view,
                                  const sharq_fp4_view *w_dense_view, int64_t m, int64_t n,
                                  int64_t k, uint16_t *y_bf16, int64_t ld_y,
                                  sharq_gemm_variant variant, void *stream);

/*
 * Grouped dual GEMM: the expert GEMMs of a mixture-of-experts layer in one
 * launch (each expert's product is sharq_dual_gemm's, abstract, sentences 4
 * and 5).  The activations are prepared once per token (sparse, resid:
 * `tokens` rows, sparse->dense_codes required); grouped row i of group e,
 * group_offsets[e] <= i < group_offsets[e + 1], is activation row
 * row_index[i] (row i itself when row_index is NULL) and meets group e's
 * weight, rows e n .. e n + n - 1 of the stacked payload w_*_view (groups n
 * rows; the two views as in sharq_dual_gemm).  Y [rows, n] (fp32, ld_y):
 * grouped row i of Y is that row's dual GEMM.
 * group_offsets (int64, groups + 1 entries) and row_index (int32, rows
 * entries) are DEVICE arrays and are not read on the host: the group sizes
 * may come from routing on the device.  The offsets must be nondecreasing
 * from 0 to rows and the indices in [0, tokens); the kernel clamps offsets to
 * [0, rows], so no value in them makes it write outside Y (an out-of-range
 * index reads zeros or another row's data).
 * MXFP4 only.  Requirements: 1 <= groups <= 256; tokens >= 1; rows >= 0 (0:
 * nothing to do); rows <= tokens without row_index; n >= 1; k >= 128,
 * k % 128 == 0; ld_y >= n; y 4-byte, group_offsets 8-byte, row_index 4-byte
 * aligned; the views as sharq_dual_gemm requires for `tokens` activation
 * rows and groups n weight rows.
 */
sharq_status sharq_grouped_dual_gemm(sharq_format fmt, const sharq_fp4_view *sparse,
                                     const sharq_fp4_view *resid, int64_t tokens,
                                     const int32_t *row_index, const int64_t *group_offsets,
                                     int64_t groups, int64_t rows,
                                     const sharq_fp4_view *w_sparse_view,
                                     const sharq_fp4_view *w_dense_view, int64_t n, int64_t k,
                                     float *y, int64_t ld_y, void *stream);

/*
 * The grouped form of sharq_dual_gemm_silu_prepare: a mixture-of-experts
 * layer's gate+up expert GEMMs (as sharq_grouped_dual_gemm: grouped row i of
 * group e is activation row row_index[i], or i, and meets group e's weight)
 * with SiLU(gate) * up and the down projections' preparation in the
 * epilogue.  Group e's weight is rows e 2 inter .. (e + 1) 2 inter - 1 of the
 * stacked payload: inter gate rows, then inter up rows.  Writes the
 * preparation of x [rows, inter] (grouped rows; x as in
 * sharq_dual_gemm_silu_prepare) to sparse_out and resid_out; byte for byte
 * what sharq_grouped_dual_gemm followed by sharq_prepare_silu_mul on the two
 * halves of its Y writes.
 * MXFP4 only.  Requirements: as sharq_grouped_dual_gemm with n = 2 inter,
 * inter >= 128 and inter % 128 == 0, and for the outputs as
 * sharq_dual_gemm_silu_prepare with rows rows (rows == 0: nothing to do).
 */
sharq_status sharq_grouped_dual_gemm_silu_prepare(
    sharq_format fmt, const sharq_fp4_view *sparse, const sharq_fp4_view *resid, int64_t tokens,
    const int32_t *row_index, const int64_t *group_offsets, int64_t groups, int64_t rows,
    const sharq_fp4_view *w_sparse_view, const sharq_fp4_view *w_dense_view, int64_t inter,
    int64_t k, const sharq_fp4_view *sparse_out, const sharq_fp4_view *resid_out, void *stream);

/* Bytes of one packed array (`which` = SHARQ_BYTES_*) for `rows` rows of length k; 0 if invalid. */
size_t sharq_bytes(sharq_format fmt, int which, int64_t rows, int64_t k);

/* Static, NUL-terminated description of a status code. */
const char *sharq_status_str(sharq_status status);

/* ABI version of this header (increments on any incompatible change). */
int sharq_abi_version(void);

#define SHARQ_ABI_VERSION 11

#ifdef __cplusplus
}
#endif

#endif /* SHARQ_H */
