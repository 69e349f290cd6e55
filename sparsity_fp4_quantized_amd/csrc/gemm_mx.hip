// Dual-path MXFP4 GEMM of the SharQ path, for gfx950.
//
// "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
// Inference" (arXiv:2606.26587), abstract, sentence 4 (a sparse FP4 GEMM on
// the backbone and a dense FP4 GEMM on the residual) and sentence 5 (both
// read one FP4 weight payload through path-specific scale views):
//
//   Y = deq(backbone) W^T + deq(residual) W^T,   fp32 accumulate, fp32 out.
//
// Both paths run on the CDNA4 block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 (E2M1) A and B operands and one
// E8M0 scale per 32 k per row and per column.  gfx950 has no structured-sparse
// MFMA for FP4 operands, so the 2:4 backbone is expanded to dense FP4 (zeros
// at the dropped positions) while it is staged into LDS.  Each K step stages
// the W tile once and feeds it to the MFMAs of both paths, which accumulate
// into the same registers.
//
// Operand layout of the 32x32x64 FP4 MFMA (lane l, h = l / 32): A row l % 32
// and B column l % 32, 32 consecutive k (16 bytes) per lane and MFMA; the E8M0
// scale of that lane's 32 k comes from the lane's scale register.  Within a
// 128-k step, lane half h takes the k blocks 2h (first MFMA) and 2h + 1
// (second MFMA); A and B use the same assignment, so the dot products are
// unchanged.
#include "fp4_device.h"
#include "kernels.h"

namespace sharq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kStride = 80;   // LDS bytes per tile row: 64 bytes of codes + 16 pad

__device__ __forceinline__ v8i as_operand(uint4 v) {
  v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

// Expand eight 2:4 groups (8 code bytes, 4 meta bytes) into 32 dense codes.
__device__ __forceinline__ void expand8(uint2 codes, uint32_t meta, uint32_t out[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      int g = 2 * q + gg;
      uint32_t cb = ((g < 4 ? codes.x : codes.y) >> (8 * (g & 3))) & 0xFFu;
      uint32_t nib = (meta >> (4 * g)) & 15u;
      uint32_t i0 = nib & 3u, i1 = nib >> 2;
      uint32_t d16 = ((cb & 15u) << (4u * i0)) | ((cb >> 4) << (4u * i1));
      word |= d16 << (16 * gg);
    }
    out[q] = word;
  }
}

template <bool kDenseExpanded>
__global__ __launch_bounds__(256) void dual_gemm_mx_kernel(GemmArgs a) {
  __shared__ __align__(16) uint8_t lds_as[BM * kStride];
  __shared__ __align__(16) uint8_t lds_ar[BM * kStride];
  __shared__ __align__(16) uint8_t lds_w[BN * kStride];
  __shared__ uint32_t lds_sas[BM], lds_sar[BM], lds_sws[BN], lds_swd[BN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int h = lane >> 5, li = lane & 31;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int ksteps = (int)(a.k / BK);
  for (int kt = 0; kt < ksteps; ++kt) {
    // ---- global -> LDS
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      int c = tid + 256 * j, row = c >> 2, part = c & 3;
      int64_t gm = m0 + row, gn = n0 + row;
      uint4 vr = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
      if (gm < a.m)
        vr = *reinterpret_cast<const uint4 *>(a.r_codes + gm * a.ld_rc + kt * 64 + part * 16);
      if (gn < a.n)
        vw = *reinterpret_cast<const uint4 *>(a.w_codes + gn * a.ld_wc + kt * 64 + part * 16);
      *reinterpret_cast<uint4 *>(lds_ar + row * kStride + part * 16) = vr;
      *reinterpret_cast<uint4 *>(lds_w + row * kStride + part * 16) = vw;
      if (kDenseExpanded) {
        uint4 vs = make_uint4(0, 0, 0, 0);
        if (gm < a.m)
          vs = *reinterpret_cast<const uint4 *>(a.s_dense + gm * a.ld_sd + kt * 64 + part * 16);
        *reinterpret_cast<uint4 *>(lds_as + row * kStride + part * 16) = vs;
      }
    }
    if (!kDenseExpanded) {
      // two threads per row, 16 groups (16 code bytes, 8 meta bytes) each
      int row = tid >> 1, half = tid & 1;
      int64_t gm = m0 + row;
      uint4 cv = make_uint4(0, 0, 0, 0);
      uint2 mv = make_uint2(0x44444444u, 0x44444444u);
      if (gm < a.m) {
        cv = *reinterpret_cast<const uint4 *>(a.s_codes + gm * a.ld_sc + kt * 32 + half * 16);
        mv = *reinterpret_cast<const uint2 *>(a.meta + gm * a.ld_meta + kt * 16 + half * 8);
      }
      uint32_t d0[4], d1[4];
      expand8(make_uint2(cv.x, cv.y), mv.x, d0);
      expand8(make_uint2(cv.z, cv.w), mv.y, d1);
      uint8_t *dst = lds_as + row * kStride + half * 32;
      *reinterpret_cast<uint4 *>(dst) = make_uint4(d0[0], d0[1], d0[2], d0[3]);
      *reinterpret_cast<uint4 *>(dst + 16) = make_uint4(d1[0], d1[1], d1[2], d1[3]);
    }
    if (tid < BM) {
      int64_t gm = m0 + tid;
      uint32_t ss = 0, sr = 0;
      if (gm < a.m) {
        ss = *reinterpret_cast<const uint32_t *>(a.s_scales + gm * a.ld_ss + kt * 4);
        sr = *reinterpret_cast<const uint32_t *>(a.r_scales + gm * a.ld_rs + kt * 4);
      }
      lds_sas[tid] = ss;
      lds_sar[tid] = sr;
    } else {
      int row = tid - BM;
      int64_t gn = n0 + row;
      uint32_t s1 = 0, s2 = 0;
      if (gn < a.n) {
        s1 = *reinterpret_cast<const uint32_t *>(a.ws_scales + gn * a.ld_wss + kt * 4);
        s2 = *reinterpret_cast<const uint32_t *>(a.wd_scales + gn * a.ld_wds + kt * 4);
      }
      lds_sws[row] = s1;
      lds_swd[row] = s2;
    }
    __syncthreads();

    // ---- MFMA
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i fas[2], far[2], fb[2];
      int sas[2], sar[2], sws[2], swd[2];
      const int off = h * 32 + s * 16, sh = 8 * (2 * h + s);
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        int r = wm * 64 + it * 32 + li;
        fas[it] = as_operand(*reinterpret_cast<const uint4 *>(lds_as + r * kStride + off));
        far[it] = as_operand(*reinterpret_cast<const uint4 *>(lds_ar + r * kStride + off));
        sas[it] = (int)((lds_sas[r] >> sh) & 0xFFu);
        sar[it] = (int)((lds_sar[r] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        int r = wn * 64 + jt * 32 + li;
        fb[jt] = as_operand(*reinterpret_cast<const uint4 *>(lds_w + r * kStride + off));
        sws[jt] = (int)((lds_sws[r] >> sh) & 0xFFu);
        swd[jt] = (int)((lds_swd[r] >> sh) & 0xFFu);
      }
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          acc[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fas[it], fb[jt], acc[it][jt], 4, 4, 0, sas[it], 0, sws[jt]);
          acc[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              far[it], fb[jt], acc[it][jt], 4, 4, 0, sar[it], 0, swd[jt]);
        }
    }
    __syncthreads();
  }

  // ---- epilogue: lane l holds column l % 32, rows 8 (r / 4) + 4 h + r % 4
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      int64_t col = n0 + wn * 64 + jt * 32 + li;
      if (col >= a.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t row = m0 + wm * 64 + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < a.m) a.y[row * a.ld_y + col] = acc[it][jt][r];
      }
    }
}

}  // namespace

hipError_t launch_dual_gemm_mx(const GemmArgs &a, bool dense_expanded, hipStream_t s) {
  dim3 grid((unsigned)((a.n + BN - 1) / BN), (unsigned)((a.m + BM - 1) / BM)), block(256);
  if (dense_expanded)
    dual_gemm_mx_kernel<true><<<grid, block, 0, s>>>(a);
  else
    dual_gemm_mx_kernel<false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sharq
