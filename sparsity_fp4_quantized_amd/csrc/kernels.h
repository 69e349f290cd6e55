// Internal launch interface between the C ABI (sharq_abi.cpp) and the HIP
// kernels.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

struct PrepArgs {
  const uint16_t *x;
  int64_t ld_x, m, k;
  const uint16_t *gamma;   // nullptr: no normalization
  float eps;
  uint8_t *s_codes;  int64_t ld_sc;
  uint8_t *meta;     int64_t ld_meta;
  uint8_t *s_scales; int64_t ld_ss;
  uint8_t *r_codes;  int64_t ld_rc;
  uint8_t *r_scales; int64_t ld_rs;
  uint8_t *s_dense;  int64_t ld_sd;   // optional
  float *tensor_scale;                // NVFP4: [0] receives the tensor scale
  int s_ksm, r_ksm;                   // backbone / residual view k-step-major (every array)
  // residual add in front of the norm (MXFP4 with normalization only):
  // x = bf16(x + add), written to x_out, then prepared; add == nullptr: none
  const uint16_t *add = nullptr;  int64_t ld_add = 0;
  uint16_t *x_out = nullptr;      int64_t ld_xout = 0;
  // SiLU(gate) * up in front of the preparation (MXFP4, no norm): fp32 gate
  // and up [m, k] replace x
  const float *gate = nullptr;    int64_t ld_gate = 0;
  const float *up = nullptr;      int64_t ld_up = 0;
  // NVFP4: where the tensor amax passes reduce (tensor_scale + 1, or the
  // allocation-free entry point's static workspace)
  float *amax = nullptr;
  // fl32(1 / k), set by the preparation's launcher for the row mean
  float inv_k = 0.0f;
};

struct QuantArgs {
  const uint16_t *w;
  int64_t ld_w, n, k;
  uint8_t *codes;  int64_t ld_c;
  uint8_t *scales; int64_t ld_s;
  float *tensor_scale;                // NVFP4
  int ksm;                            // codes and scales k-step-major
};

struct GemmArgs {
  const uint8_t *s_codes;  int64_t ld_sc;   // 2:4 backbone [m, k/4]
  const uint8_t *meta;     int64_t ld_meta; // [m, k/8]
  const uint8_t *s_dense;  int64_t ld_sd;   // dense backbone [m, k/2] (DENSE_EXPANDED)
  const uint8_t *s_scales; int64_t ld_ss;
  const uint8_t *r_codes;  int64_t ld_rc;
  const uint8_t *r_scales; int64_t ld_rs;
  const uint8_t *w_codes;  int64_t ld_wc;
  const uint8_t *ws_scales; int64_t ld_wss; // sparse-path scale view of W
  const uint8_t *wd_scales; int64_t ld_wds; // dense-path scale view of W
  const float *a_tensor_scale;              // NVFP4
  const float *w_tensor_scale;              // NVFP4
  float *y;                int64_t ld_y;      // fp32 Y [m, n] (null when y16 is set)
  int64_t m, n, k;
  int s_ksm, r_ksm, w_ksm;   // per operand (codes, meta, dense view, scales): k-step-major
  // grouped GEMM (mixture of experts): m = grouped rows in total; grouped row
  // i of group e (group_off[e] <= i < group_off[e + 1], device array) is
  // activation row row_index[i] (i when row_index is null) of `tokens`
  // activation rows, and meets group e's weight, rows e n .. e n + n - 1
  const int32_t *row_index = nullptr;
  const int64_t *group_off = nullptr;
  int64_t groups = 0, tokens = 0;
  // bf16 Y [m, n] (row stride ld_y elements) in place of y: each value the
  // bf16 rounding (nearest even) of the fp32 value y would receive
  uint16_t *y16 = nullptr;
};

// Offset of the bytes of row r in 128-k step t of an operand array with `bps`
// bytes per row and step: row-major (ld bytes per row) or k-step-major (ld
// rows per step).
__host__ __device__ inline int64_t arr_off(int64_t r, int64_t t, int64_t ld, int ksm, int64_t bps) {
  return ksm ? (t * ld + r) * bps : r * ld + t * bps;
}

hipError_t launch_prepare_mx(const PrepArgs &a, hipStream_t s);
hipError_t launch_prepare_silu_mx(const PrepArgs &a, hipStream_t s);
hipError_t launch_prepare_nv(const PrepArgs &a, hipStream_t s);
// sharq_prepare_noalloc's launches: a.amax is set to this device's static
// workspace (its address taken once per device); MXFP4 uses no workspace
hipError_t launch_prepare_noalloc(PrepArgs a, int fmt, hipStream_t s);
hipError_t launch_quantize_weight_mx(const QuantArgs &a, hipStream_t s);
hipError_t launch_quantize_weight_nv(const QuantArgs &a, hipStream_t s);
hipError_t launch_dual_gemm_mx(const GemmArgs &a, bool dense_expanded, hipStream_t s);
// the 2:4 backbone (codes + meta) on the structured-sparse FP8 MFMA, rebased
// per tile; tiles that cannot be rebased exactly expand it to dense FP4
hipError_t launch_dual_gemm_mx_fp8sp(const GemmArgs &a, hipStream_t s);
hipError_t launch_grouped_dual_gemm_mx(const GemmArgs &a, hipStream_t s);
// gate+up dual GEMM (a.n = 2 i: i gate rows, then i up rows of W; i % 128 == 0)
// with x = bf16(silu(gate) * up) prepared into p's outputs ([a.m, i], no norm)
hipError_t launch_dual_gemm_silu_prep_mx(const GemmArgs &a, const PrepArgs &p, hipStream_t s);
// the same over the groups of a grouped GEMM (each group's W: a.n rows, gate
// then up); p's outputs have a.m (grouped) rows
hipError_t launch_grouped_dual_gemm_silu_prep_mx(const GemmArgs &a, const PrepArgs &p, hipStream_t s);
hipError_t launch_dual_gemm_nv(const GemmArgs &a, int variant, hipStream_t s);

}  // namespace sharq
