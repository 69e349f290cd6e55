// Fused preparation operator of the SharQ path, for gfx950.
//
// "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
// Inference" (arXiv:2606.26587), abstract, sentence 3 (input-adaptive N:M
// mask, FP4 backbone, residual against the quantized backbone) and sentence 5
// (one fused operator that also absorbs the layer normalization).
//
// Work split: one lane owns one 32-element block of a row (one MXFP4 scale
// block, eight 2:4 groups, or two NVFP4 blocks), so each lane reads 64
// contiguous bytes and writes whole words of every output.  With RMSNorm a
// workgroup holds R whole rows (R = 1, 2 or 4 rows per wavefront, a row over
// W wavefronts); the sum of squares follows a fixed binary tree: a tree over
// the 32 squares inside the lane, a xor butterfly across the lanes of the
// row, and a tree over the W wavefronts' sums in LDS (missing leaves +0).
// That is the pairwise tree over 2^ceil(log2 K) leaves, whatever R and W.
// Without normalization the blocks are independent and the grid is flat.
//
// Fused neighbours (the steps next to the preparation in a decoder layer):
// the norm kernel's ADD variant adds the residual stream and the sublayer
// output first (sharq_prepare_residual), and prep_silu_kernel forms SiLU(gate)
// * up from the gate+up projection's fp32 output (sharq_prepare_silu_mul).
//
// MXFP4 element and scale conversions use the gfx950 instructions
// v_cvt_scalef32_pk_fp4_{bf16,f32} (round to nearest even, saturating, sign
// of zero kept; the scale operand acts as 2^(E8M0 byte - 127), also for byte 0)
// and v_cvt_scalef32_pk_f32_fp4 (exact dequantization).  The NVFP4-style path
// divides by its non-power-of-two scale in IEEE fp32 first and converts at
// scale 1.
#include <mutex>
#include <type_traits>

#include "fp4_device.h"
#include "kernels.h"
#include "prep_block.h"

namespace sharq {
namespace {

constexpr int kMaxWavesPerRow = 8;     // K <= 16384 with normalization

// ---------------------------------------------------------------- helpers

// 32 bf16 values (64 bytes) as four 16-byte loads.  Plain loads: a
// wavefront's four loads cover each 128-byte line between them, and the L1
// serves the later ones; non-temporal loads (which skip it) fetched every line
// again for each load and made the preparation 10-28% slower.
__device__ __forceinline__ void load32(const uint16_t *p, uint32_t w[16]) {
  const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 t = q[i];
    w[4 * i + 0] = t.x;
    w[4 * i + 1] = t.y;
    w[4 * i + 2] = t.z;
    w[4 * i + 3] = t.w;
  }
}

// two fp32 -> bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 v = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Tree sum of the 32 squares of a block (adjacent pairs at every level).
__device__ __forceinline__ float block_sumsq(const float f[32]) {
  float q[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) q[i] = f[i] * f[i];
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) q[i] = q[2 * i] + q[2 * i + 1];
  }
  return q[0];
}

// Butterfly over the 64 lanes: step j adds lane l ^ 2^j, so every lane ends
// with the pairwise tree sum of the 64 values (fp32 addition commutes).
template <int XOR>
__device__ __forceinline__ float swz_xor(float v) {
  // ds_swizzle bit-mask mode inside 32-lane halves: and 0x1F, or 0, xor XOR
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (XOR << 10)));
}

// Sum over each aligned group of L lanes (L a power of two <= 64), as a
// perfect binary tree of adjacent pairs; every lane of a group gets the sum.
template <int L>
__device__ __forceinline__ float lane_tree_sum(float v) {
  if (L >= 2) v = v + swz_xor<1>(v);
  if (L >= 4) v = v + swz_xor<2>(v);
  if (L >= 8) v = v + swz_xor<4>(v);
  if (L >= 16) v = v + swz_xor<8>(v);
  if (L >= 32) v = v + swz_xor<16>(v);
  if (L >= 64)
    v = v + __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) & 63) << 2,
                                                        __float_as_int(v)));
  return v;
}

__device__ __forceinline__ float wave_tree_sum(float v) {
  v = v + swz_xor<1>(v);
  v = v + swz_xor<2>(v);
  v = v + swz_xor<4>(v);
  v = v + swz_xor<8>(v);
  v = v + swz_xor<16>(v);
  // lane l ^ 32: the other half of the wavefront
  v = v + __int_as_float(__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) & 63) << 2,
                                                      __float_as_int(v)));
  return v;
}

// ---------------------------------------------------------------- NVFP4 block

// E2M1 codes of fl32(v / S) for 32 values (two 16-blocks with scales S[0], S[1]),
// signed zeros when S == 0; packed two per byte.
__device__ __forceinline__ void nv_codes(const float v[32], const float S[2], uint32_t out[4]) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  float y[2];
  bool fast[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    fast[b] = S[b] >= 0x1p-100f && S[b] <= 0x1p100f;
    y[b] = 1.0f / S[b];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float s = S[i >> 3];
    float t0 = v[2 * i], t1 = v[2 * i + 1];
    // S == 0: keep only the sign (the conversion of +-0 keeps it)
    if (fast[i >> 3]) {
      t0 = div_rn(t0, s, y[i >> 3]);
      t1 = div_rn(t1, s, y[i >> 3]);
    } else {
      t0 = s == 0.0f ? __uint_as_float(__float_as_uint(t0) & 0x80000000u) : t0 / s;
      t1 = s == 0.0f ? __uint_as_float(__float_as_uint(t1) & 0x80000000u) : t1 / s;
    }
    uint32_t &x = w[i >> 2];
    switch (i & 3) {
      case 0: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, t0, t1, 1.0f, 0); break;
      case 1: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, t0, t1, 1.0f, 1); break;
      case 2: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, t0, t1, 1.0f, 2); break;
      default: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, t0, t1, 1.0f, 3); break;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = w[q];
}

// Block scale byte and effective scale S = fl32(e4m3(byte) * s_t).
__device__ __forceinline__ uint32_t nv_scale(float amax, float s_t, float &S) {
  float ratio = amax / (6.0f * s_t);
  uint32_t sb = e4m3_encode_pos(ratio);
  S = e4m3_value(sb) * s_t;
  return sb;
}

__device__ __forceinline__ void quantize_block_nv(const float xf[32], float s_t, BlockOut &o) {
  MaskOut mk;
  mask_block(xf, mk);
  o.meta = mk.meta;

  float S[2];
  uint32_t sb0, sb1;
  {
    uint32_t a0 = 0, a1 = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) a0 = max(a0, mk.top[g]);
#pragma unroll
    for (int g = 4; g < 8; ++g) a1 = max(a1, mk.top[g]);
    sb0 = nv_scale(__uint_as_float(a0 & 0x7FFF0000u), s_t, S[0]);
    sb1 = nv_scale(__uint_as_float(a1 & 0x7FFF0000u), s_t, S[1]);
  }
  o.s_scale = sb0 | (sb1 << 8);

  uint32_t full[4];
  nv_codes(xf, S, full);
  // keep mask per group from the two kept indices
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int g = 2 * q + h;
      uint32_t s0 = 12u - 4u * mk.umax[g], s1 = 12u - 4u * mk.umin[g];
      m2[h] = (0xFu << s0) | (0xFu << s1);
    }
    o.s_dense[q] = full[q] & (m2[0] | (m2[1] << 16));
  }
  // compressed bytes: nibbles at i0 and i1 of each group
  uint32_t comp[2] = {0u, 0u};
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t d16 = (o.s_dense[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
    uint32_t s0 = 12u - 4u * mk.umax[g], s1 = 12u - 4u * mk.umin[g];
    uint32_t byte = ((d16 >> s0) & 15u) | (((d16 >> s1) & 15u) << 4);
    comp[g >> 2] |= byte << (8 * (g & 3));
  }
  o.s_comp[0] = comp[0];
  o.s_comp[1] = comp[1];

  // residual: R = x_n - fl32(value * S)
  float res[32];
  float ra0 = 0.0f, ra1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f32x2 d;
    switch (i & 3) {
      case 0: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], 1.0f, 0); break;
      case 1: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], 1.0f, 1); break;
      case 2: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], 1.0f, 2); break;
      default: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], 1.0f, 3); break;
    }
    const float s = S[i >> 3];
    res[2 * i] = xf[2 * i] - d[0] * s;
    res[2 * i + 1] = xf[2 * i + 1] - d[1] * s;
    float m = fmaxf(fabsf(res[2 * i]), fabsf(res[2 * i + 1]));
    if (i < 8) ra0 = fmaxf(ra0, m); else ra1 = fmaxf(ra1, m);
  }
  float R[2];
  uint32_t rb0 = nv_scale(ra0, s_t, R[0]);
  uint32_t rb1 = nv_scale(ra1, s_t, R[1]);
  o.r_scale = rb0 | (rb1 << 8);
  nv_codes(res, R, o.r_codes);
}

// ---------------------------------------------------------------- stores

// s_t = fl32(amax / 2688) (1 when amax = 0), from the reduced tensor amax
__device__ __forceinline__ float nv_tensor_scale(const float *amax_slot) {
  float amax = *amax_slot;
  return amax == 0.0f ? 1.0f : amax / 2688.0f;
}

// ---------------------------------------------------------------- row RMS

// Row reduction: `s` is the lane's block sum of squares (0 for lanes past the
// row end); every thread of the workgroup calls this.  Returns
// r = 1 / sqrt(ss / k + eps) of the lane's row.
// `buf` alternates between calls of one loop, so that a wavefront writing the
// next row's partial sums never overwrites values another is still reading.
template <int WPR>
__device__ __forceinline__ float row_rms(float s, int riw, int wir, int64_t k, float eps, int buf = 0) {
  __shared__ float part[2][4 * kMaxWavesPerRow];
  s = wave_tree_sum(s);
  if ((threadIdx.x & 63) == 0) part[buf][riw * kMaxWavesPerRow + wir] = s;
  __syncthreads();
  float c[kMaxWavesPerRow];
#pragma unroll
  for (int i = 0; i < kMaxWavesPerRow; ++i) c[i] = i < WPR ? part[buf][riw * kMaxWavesPerRow + i] : 0.0f;
#pragma unroll
  for (int w = kMaxWavesPerRow / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) c[i] = c[2 * i] + c[2 * i + 1];
  }
  float mean = c[0] / (float)k;
  float var = mean + eps;
  float sd = __builtin_sqrtf(var);
  return 1.0f / sd;
}

// x_n = bf16((x * r) * gamma): returns the bf16 pairs and overwrites xf with x_n.
__device__ __forceinline__ void normalize32(float xf[32], uint32_t xw[16], const float gf[32],
                                            float r) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float lo = (xf[2 * i] * r) * gf[2 * i];
    float hi = (xf[2 * i + 1] * r) * gf[2 * i + 1];
    xw[i] = pack_bf16x2(lo, hi);
    xf[2 * i] = bf16_lo(xw[i]);
    xf[2 * i + 1] = bf16_hi(xw[i]);
  }
}

__device__ __forceinline__ void normalize32(float xf[32], uint32_t xw[16], const uint16_t *g,
                                            float r) {
  uint32_t gw[16];
  float gf[32];
  load32(g, gw);
  unpack32(gw, gf);
  normalize32(xf, xw, gf, r);
}

// base + uniform + lane bytes: the uniform part stays in scalar registers and
// the access takes a 32-bit vector offset
template <class T>
__device__ __forceinline__ T *at_bytes(T *base, int64_t uniform_bytes, uint32_t lane_bytes) {
  using B = typename std::conditional<std::is_const<T>::value, const uint8_t, uint8_t>::type;
  return reinterpret_cast<T *>(reinterpret_cast<B *>(base) + uniform_bytes + lane_bytes);
}

__device__ __forceinline__ float row_mean(float ss, const PrepArgs &a) {
  return row_mean_of(ss, (float)a.k, a.inv_k);
}

// ---------------------------------------------------------------- kernels

// A lane's 32 bf16 values as four 16-byte stores.  Plain stores: each one
// writes a quarter of 32 lines, and the L2 merges the four quarters before the
// lines leave it; non-temporal, the partial lines went out one by one (the
// residual-add preparation took 20.9 against 16.5 us on the qkv shape).
__device__ __forceinline__ void store32(uint16_t *p, const uint32_t w[16]) {
  u32x4 *q = reinterpret_cast<u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
}

// Workgroup = R rows x W wavefronts: lane l of wavefront w takes row rl =
// l / L (L = 64 / R lanes per row) and block b = w L + l % L, so a wavefront
// stores R consecutive rows of each 128-k step next to each other in the
// k-step-major layout (R = 1 keeps a row's blocks contiguous for the
// row-major layout).
// The row's sum of squares is the oracle's perfect binary tree: the lane's 32
// values, then adjacent lanes of the row (butterfly over L lanes), then the W
// wavefronts in LDS (padded to a power of two with zeros).  Lanes past the row
// end (or past the last row) load a valid block of X and contribute +0; they
// store nothing.  ADD: the residual add in front of the norm, x = bf16(x +
// add) (the binary32 sum rounded to nearest even), stored to x_out as the new
// residual stream and prepared in place of X; x_out may be X itself or `add`,
// since every lane reads its block before it writes it.
// Addresses: wavefront-uniform 64-bit bases plus 32-bit lane offsets (the
// host bounds the row strides of the bf16 arrays below 2^28 elements and every
// output array below 4 GiB); on the qkv shape this, the median-of-three in the
// mask and the row mean without an IEEE division took the VALU instructions
// per wavefront from 723 to 666 (SQ_INSTS_VALU) and the kernel time down by
// about 5%.  (Two row groups per workgroup, the second group's loads issued
// during the first group's quantization, ran at two wavefronts per SIMD and
// was 4% slower than this; two blocks of one row per lane, 13% slower.)
template <int FMT, int R, int W, bool ADD>
__global__ __launch_bounds__(64 * W) void prep_norm_kernel(PrepArgs a) {
  constexpr int L = 64 / R;
  __shared__ float part[R][W];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t rl = (uint32_t)lane / L, lb = (uint32_t)lane % L;
  const int64_t rs = (int64_t)blockIdx.x * R;    // the group's first row (< m)
  const bool row_ok = rs + rl < a.m;
  const int64_t nblk = a.k / 32;
  const int64_t b0 = (int64_t)wave * L;          // the wavefront's first block (uniform)
  const int64_t b = b0 + lb;
  const bool has = row_ok && b < nblk;
  // bf16 arrays: byte offset 2 ld row + 64 b; lanes past the row end read
  // block 0, rows past the last one the group's first row
  const uint32_t vb = b < nblk ? 64u * (uint32_t)b : 0u;
  const uint32_t rlx = row_ok ? rl : 0u;
  uint32_t xw[16], gw[16];
  float xf[32];
  load32(at_bytes(a.x, 2 * rs * a.ld_x, rlx * (2u * (uint32_t)a.ld_x) + vb), xw);
  // gamma's loads go out with X's, so that they land during the row
  // reduction rather than after it
  load32(at_bytes(a.gamma, 0, vb), gw);
  if (ADD) {
    uint32_t ow[16];
    load32(at_bytes(a.add, 2 * rs * a.ld_add, rlx * (2u * (uint32_t)a.ld_add) + vb), ow);
    float of[32];
    unpack32(xw, xf);
    unpack32(ow, of);
#pragma unroll
    for (int i = 0; i < 16; ++i) xw[i] = pack_bf16x2(xf[2 * i] + of[2 * i], xf[2 * i + 1] + of[2 * i + 1]);
    if (has) store32(at_bytes(a.x_out, 2 * rs * a.ld_xout, rl * (2u * (uint32_t)a.ld_xout) + vb), xw);
  }
  unpack32(xw, xf);
  float r;
  if constexpr (FMT == 1) {
    // NVFP4: the tensor-amax pre-pass computed the row's r (the same tree and
    // steps) and left it in the first 4 bytes of the row's residual codes;
    // every lane has read it before the barrier, and only then does the
    // row's first block overwrite it
    r = *reinterpret_cast<const float *>(a.r_codes + arr_off(rs + rlx, 0, a.ld_rc, a.r_ksm, 64));
    __syncthreads();
  } else {
    const float s = lane_tree_sum<L>(has ? block_sumsq(xf) : 0.0f);
    if (lb == 0) part[rl][wave] = s;
    __syncthreads();
    float c[W];
#pragma unroll
    for (int i = 0; i < W; ++i) c[i] = part[rl][i];
#pragma unroll
    for (int w = W / 2; w >= 1; w >>= 1) {
#pragma unroll
      for (int i = 0; i < w; ++i) c[i] = c[2 * i] + c[2 * i + 1];
    }
    r = 1.0f / __builtin_sqrtf(row_mean(c[0], a) + a.eps);
  }
  if (!has) return;
  {
    float gf[32];
    unpack32(gw, gf);
    normalize32(xf, xw, gf, r);
  }
  BlockOut o;
  if (FMT == 0) {
    quantize_block_mx(xw, xf, o);
  } else {
    const float s_t = nv_tensor_scale(a.amax);
    if (rs + rl == 0 && b == 0) a.tensor_scale[0] = s_t;
    quantize_block_nv(xf, s_t, o);
  }
  store_block_at<FMT, (R >= 4)>(a, rs, b0 / 4, lane_offsets<FMT>(a, rl, lb >> 2, lb & 3), o);
}

// Few rows (decode: m <= 32, MXFP4 with RMSNorm, K <= 8192).  With one lane
// per 32-element block a row is only K / 32 lanes: the GPU runs a few dozen
// wavefronts, and each lane's chain of about 660 dependent instructions sets
// the time.  Here four lanes share a block, eight consecutive k each (two 2:4
// groups): the four lanes of a quad hold one block, and its two block maxima
// meet through DPP quad permutes.  One workgroup per row, W wavefronts.
// Every value comes from the same steps as in the one-lane-per-block kernels:
// the sum of squares by the same tree (the lane's 8 squares, a xor butterfly
// over the wavefront, the wavefronts' sums in LDS, missing leaves +0), the
// mask by the same keys, the codes and scales by the same conversions.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t quad_max_all(uint32_t v) {
  v = quad_max<0xB1>(v);   // quad_perm [1, 0, 3, 2]: the lane's neighbour
  return quad_max<0x4E>(v);  // quad_perm [2, 3, 0, 1]: the other pair
}

template <int W>
__global__ __launch_bounds__(64 * W) void prep_norm_quad_kernel(PrepArgs a) {
  __shared__ float part[W];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t t = threadIdx.x;                 // the lane's 8-element slice of the row
  const int64_t row = blockIdx.x;
  const bool has = (int64_t)t < a.k / 8;          // whole quads: k % 32 == 0
  const uint32_t vb = has ? 16u * t : 0u;         // lanes past the row end read slice 0
  const u32x4 xv = *reinterpret_cast<const u32x4 *>(at_bytes(a.x, 2 * row * a.ld_x, vb));
  const u32x4 gv = *reinterpret_cast<const u32x4 *>(at_bytes(a.gamma, 0, vb));
  uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
  float xf[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xf[2 * i] = bf16_lo(xw[i]);
    xf[2 * i + 1] = bf16_hi(xw[i]);
  }
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = xf[i] * xf[i];
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) q[i] = q[2 * i] + q[2 * i + 1];
  }
  const float s = wave_tree_sum(has ? q[0] : 0.0f);
  if ((threadIdx.x & 63) == 0) part[wave] = s;
  __syncthreads();
  float c[W];
#pragma unroll
  for (int i = 0; i < W; ++i) c[i] = part[i];
#pragma unroll
  for (int w = W / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) c[i] = c[2 * i] + c[2 * i + 1];
  }
  const float r = 1.0f / __builtin_sqrtf(row_mean(c[0], a) + a.eps);
  if (!has) return;   // whole quads leave together

  // x_n = bf16((x r) gamma)
  const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xw[i] = pack_bf16x2((xf[2 * i] * r) * bf16_lo(gw[i]), (xf[2 * i + 1] * r) * bf16_hi(gw[i]));
    xf[2 * i] = bf16_lo(xw[i]);
    xf[2 * i + 1] = bf16_hi(xw[i]);
  }

  // 2:4 mask of the lane's two groups (the keys of mask_block)
  uint32_t top[2], umax[2], umin[2], meta = 0;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t k0 = (__float_as_uint(xf[4 * g + 0]) & 0x7FFF0000u) | 3u;
    const uint32_t k1 = (__float_as_uint(xf[4 * g + 1]) & 0x7FFF0000u) | 2u;
    const uint32_t k2 = (__float_as_uint(xf[4 * g + 2]) & 0x7FFF0000u) | 1u;
    const uint32_t k3 = (__float_as_uint(xf[4 * g + 3]) & 0x7FFF0000u);
    const uint32_t t3 = max(max(k0, k1), k2);
    const uint32_t md = med3_u32(k0, k1, k2);
    top[g] = max(t3, k3);
    const uint32_t second = max(md, min(t3, k3));
    const uint32_t ut = top[g] & 3u, us = second & 3u;
    umax[g] = max(ut, us);
    umin[g] = min(ut, us);
    meta |= (15u - (umax[g] + (umin[g] << 2))) << (4 * g);
  }

  // backbone scale from the block amax (the quad's four lanes)
  const uint32_t am = quad_max_all(max(top[0], top[1]));
  const int ex = (int)(am >> 23);
  const uint32_t sb = ex > 2 ? (uint32_t)(ex - 2) : 0u;
  const float ss = e8m0_operand(sb);

  // compressed backbone: one byte per group
  uint32_t comp = 0u;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint32_t z = umax[g] | (umin[g] << 16);
    const uint32_t sel = 0x07060706u - __umul24(z, 0x0202u);
    const bf16x2 pv = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(xw[2 * g + 1], xw[2 * g], sel));
    comp = g == 0 ? __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(comp, pv, ss, 0)
                  : __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(comp, pv, ss, 1);
  }
  // dense backbone codes: all eight, then the dropped nibbles cleared
  uint32_t full = 0u;
  full = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(full, __builtin_bit_cast(bf16x2, xw[0]), ss, 0);
  full = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(full, __builtin_bit_cast(bf16x2, xw[1]), ss, 1);
  full = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(full, __builtin_bit_cast(bf16x2, xw[2]), ss, 2);
  full = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(full, __builtin_bit_cast(bf16x2, xw[3]), ss, 3);
  uint32_t keep = 0u;
#pragma unroll
  for (int g = 0; g < 2; ++g)
    keep |= ((0xFu << (12u - 4u * umax[g])) | (0xFu << (12u - 4u * umin[g]))) << (16 * g);
  const uint32_t dense = full & keep;

  // residual against the quantized backbone (exact in fp32), its scale from
  // the quad's amax
  float res[8];
  uint32_t ramax = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x2 d;
    switch (i) {
      case 0: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dense, ss, 0); break;
      case 1: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dense, ss, 1); break;
      case 2: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dense, ss, 2); break;
      default: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dense, ss, 3); break;
    }
    res[2 * i] = xf[2 * i] - d[0];
    res[2 * i + 1] = xf[2 * i + 1] - d[1];
    ramax = max(ramax, max(__float_as_uint(res[2 * i]) & 0x7FFFFFFFu, __float_as_uint(res[2 * i + 1]) & 0x7FFFFFFFu));
  }
  ramax = quad_max_all(ramax);
  const int rex = (int)(ramax >> 23);
  const uint32_t rb = rex > 2 ? (uint32_t)(rex - 2) : 0u;
  const float rsc = e8m0_operand(rb);
  uint32_t rc = 0u;
  rc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rc, res[0], res[1], rsc, 0);
  rc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rc, res[2], res[3], rsc, 1);
  rc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rc, res[4], res[5], rsc, 2);
  rc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(rc, res[6], res[7], rsc, 3);

  // stores: slice t is k 8t .. 8t + 7, in 128-k step t / 16
  const int64_t step = t >> 4;
  const uint32_t j = t & 15u;
  *reinterpret_cast<uint16_t *>(a.s_codes + arr_off(row, step, a.ld_sc, a.s_ksm, 32) + 2 * j) = (uint16_t)comp;
  a.meta[arr_off(row, step, a.ld_meta, a.s_ksm, 16) + j] = (uint8_t)meta;
  *reinterpret_cast<uint32_t *>(a.r_codes + arr_off(row, step, a.ld_rc, a.r_ksm, 64) + 4 * j) = rc;
  if (a.s_dense) *reinterpret_cast<uint32_t *>(a.s_dense + arr_off(row, step, a.ld_sd, a.s_ksm, 64) + 4 * j) = dense;
  if ((t & 3u) == 0u) {
    a.s_scales[arr_off(row, step, a.ld_ss, a.s_ksm, 4) + (j >> 2)] = (uint8_t)sb;
    a.r_scales[arr_off(row, step, a.ld_rs, a.r_ksm, 4) + (j >> 2)] = (uint8_t)rb;
  }
}

// No normalization: blocks are independent.  A wavefront takes R rows x
// 64 / R consecutive blocks: R = 16 (one 128-k step of 16 consecutive rows)
// makes every store of the k-step-major layout 16 rows contiguous; R = 1 (64
// blocks of one row) does the same for the row-major layout.
// Addresses as in the norm kernel: wavefront-uniform bases (the wavefront's
// first row and block) plus 32-bit lane offsets.
template <int FMT, int R>
__global__ __launch_bounds__(256) void prep_flat_kernel(PrepArgs a, uint32_t chunks) {
  constexpr int L = 64 / R;
  const uint32_t w = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t rg = w / chunks;
  const uint32_t rl = (uint32_t)lane / L, lb = (uint32_t)lane % L;
  const int64_t rs = (int64_t)rg * R, b0 = (int64_t)(w - rg * chunks) * L;   // uniform
  const int64_t row = rs + rl, b = b0 + lb;
  if (row >= a.m || b >= a.k / 32) return;
  uint32_t xw[16];
  float xf[32];
  load32(at_bytes(a.x, 2 * rs * a.ld_x + 64 * b0, rl * (2u * (uint32_t)a.ld_x) + 64u * lb), xw);
  unpack32(xw, xf);
  BlockOut o;
  if (FMT == 0) {
    quantize_block_mx(xw, xf, o);
  } else {
    float s_t = nv_tensor_scale(a.amax);
    if (row == 0 && b == 0) a.tensor_scale[0] = s_t;
    quantize_block_nv(xf, s_t, o);
  }
  store_block_at<FMT, true>(a, rs, b0 / 4, lane_offsets<FMT>(a, rl, lb >> 2, lb & 3), o);
}

// One lane per 32-k block, laid out as prep_flat_kernel's lanes: the block of
// gate and up (fp32, 128 bytes each), x = SiLU(g) * u, then the preparation
// of x without a norm.
template <int R>
__global__ __launch_bounds__(256) void prep_silu_kernel(PrepArgs a, uint32_t chunks) {
  constexpr int L = 64 / R;
  const uint32_t w = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t rg = w / chunks;
  const uint32_t rl = (uint32_t)lane / L, lb = (uint32_t)lane % L;
  const int64_t rs = (int64_t)rg * R, b0 = (int64_t)(w - rg * chunks) * L;   // uniform
  const int64_t row = rs + rl, b = b0 + lb;
  if (row >= a.m || b >= a.k / 32) return;
  const u32x4 *gp = reinterpret_cast<const u32x4 *>(
      at_bytes(a.gate, 4 * rs * a.ld_gate + 128 * b0, rl * (4u * (uint32_t)a.ld_gate) + 128u * lb));
  const u32x4 *upp = reinterpret_cast<const u32x4 *>(
      at_bytes(a.up, 4 * rs * a.ld_up + 128 * b0, rl * (4u * (uint32_t)a.ld_up) + 128u * lb));
  u32x4 gq[8], uq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    gq[i] = gp[i];
    uq[i] = upp[i];
  }
  uint32_t xw[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t lo = silu_mul_bf16(__uint_as_float(gq[i][2 * j]), __uint_as_float(uq[i][2 * j]));
      const uint32_t hi = silu_mul_bf16(__uint_as_float(gq[i][2 * j + 1]), __uint_as_float(uq[i][2 * j + 1]));
      xw[2 * i + j] = lo | (hi << 16);
    }
  }
  float xf[32];
  unpack32(xw, xf);
  BlockOut o;
  quantize_block_mx(xw, xf, o);
  store_block_at<0, true>(a, rs, b0 / 4, lane_offsets<0>(a, rl, lb >> 2, lb & 3), o);
}

// NVFP4 tensor amax of x_n.  fp32 bit patterns of non-negative values order
// like unsigned integers; each workgroup reduces its share (grid-stride) and
// issues at most one atomic max, so that few atomics meet at the one address.
__device__ __forceinline__ void block_amax_atomic(uint32_t am, float *slot) {
  __shared__ uint32_t wmax[8];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 64));
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) wmax[wave] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int i = 0; i < nw; ++i) m = max(m, wmax[i]);
    // the value only grows: skip the atomic when memory already holds >= m
    unsigned int *p = reinterpret_cast<unsigned int *>(slot);
    if (m > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, m);
  }
}

constexpr unsigned kAmaxGrid = 2048;   // workgroups of the amax passes (at most)

template <int WPR>
__global__ __launch_bounds__(512) void amax_norm_kernel(PrepArgs a) {
  constexpr int RPW = WPR <= 4 ? 4 / WPR : 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int riw = wave / WPR, wir = wave - riw * WPR;
  const int64_t nblk = a.k / 32;
  const int64_t b = (int64_t)wir * 64 + lane;
  const int64_t groups = (a.m + RPW - 1) / RPW;
  uint32_t am = 0;
  for (int64_t gi = blockIdx.x; gi < groups; gi += gridDim.x) {
    const int64_t row = gi * RPW + riw;
    const bool has = row < a.m && b < nblk;
    const int64_t lrow = row < a.m ? row : 0, lb = b < nblk ? b : 0;
    uint32_t xw[16];
    float xf[32];
    load32(a.x + lrow * a.ld_x + 32 * lb, xw);
    unpack32(xw, xf);
    float s = block_sumsq(xf);
    float r = row_rms<WPR>(has ? s : 0.0f, riw, wir, a.k, a.eps);
    // the row's r for the preparation pass, in the first 4 bytes of the row's
    // residual codes (that pass reads it before it stores the codes there)
    if (row < a.m && wir == 0 && lane == 0)
      *reinterpret_cast<float *>(a.r_codes + arr_off(row, 0, a.ld_rc, a.r_ksm, 64)) = r;
    if (has) {
      normalize32(xf, xw, a.gamma + 32 * b, r);
#pragma unroll
      for (int i = 0; i < 32; ++i) am = max(am, __float_as_uint(xf[i]) & 0x7FFFFFFFu);
    }
    __syncthreads();   // the row reduction's LDS is reused by the next row group
  }
  block_amax_atomic(am, a.amax);
}

__global__ __launch_bounds__(256) void amax_flat_kernel(const uint16_t *x, int64_t ld, int64_t m,
                                                        int64_t k, float *slot) {
  const int64_t nblk = k / 32, total = m * nblk;
  uint32_t am = 0;
  for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * 256) {
    const int64_t row = gid / nblk, b = gid - row * nblk;
    uint32_t xw[16];
    load32(x + row * ld + 32 * b, xw);
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, max(xw[i] & 0x7FFFu, (xw[i] >> 16) & 0x7FFFu));
  }
  block_amax_atomic(am << 16, slot);
}

__global__ void zero_amax_kernel(float *slot) { *slot = 0.0f; }

template <int FMT, int R, int W, bool ADD>
void launch_norm(const PrepArgs &a, hipStream_t s) {
  prep_norm_kernel<FMT, R, W, ADD><<<dim3((unsigned)((a.m + R - 1) / R)), dim3(64 * W), 0, s>>>(a);
}

template <int WPR>
void launch_amax_norm(const PrepArgs &a, hipStream_t s) {
  constexpr int RPW = WPR <= 4 ? 4 / WPR : 1;
  const unsigned groups = (unsigned)((a.m + RPW - 1) / RPW);
  amax_norm_kernel<WPR><<<dim3(min(groups, kAmaxGrid)), dim3(64 * WPR * RPW), 0, s>>>(a);
}

// W = nblk / (64 / R) wavefronts per row group, rounded up to a power of two <= 8.
template <int FMT, int R, bool ADD>
void launch_norm_w(const PrepArgs &a, int64_t nblk, hipStream_t s) {
  const int64_t w = (nblk + 64 / R - 1) / (64 / R);
  if (w <= 1) launch_norm<FMT, R, 1, ADD>(a, s);
  else if (w <= 2) launch_norm<FMT, R, 2, ADD>(a, s);
  else if (w <= 4) launch_norm<FMT, R, 4, ADD>(a, s);
  else launch_norm<FMT, R, 8, ADD>(a, s);
}

// the residual-add kernels exist for MXFP4 only (the entry point refuses NVFP4)
template <int FMT, int R>
void launch_norm_rows(const PrepArgs &a, int64_t nblk, hipStream_t s) {
  if constexpr (FMT == 0) {
    if (a.add) {
      launch_norm_w<FMT, R, true>(a, nblk, s);
      return;
    }
  }
  launch_norm_w<FMT, R, false>(a, nblk, s);
}

template <int FMT>
hipError_t launch_prepare(const PrepArgs &args, hipStream_t s) {
  PrepArgs a = args;
  a.inv_k = 1.0f / (float)a.k;   // IEEE binary32 division on the host
  const int64_t nblk = a.k / 32;
  const bool ksm = a.s_ksm != 0;
  if (FMT == 1) zero_amax_kernel<<<1, 1, 0, s>>>(a.amax);
  if (a.gamma) {
    if (FMT == 1) {
      switch ((nblk + 63) / 64) {   // wavefronts per row of the pre-pass
        case 1: launch_amax_norm<1>(a, s); break;
        case 2: launch_amax_norm<2>(a, s); break;
        case 3: launch_amax_norm<3>(a, s); break;
        case 4: launch_amax_norm<4>(a, s); break;
        case 5: launch_amax_norm<5>(a, s); break;
        case 6: launch_amax_norm<6>(a, s); break;
        case 7: launch_amax_norm<7>(a, s); break;
        default: launch_amax_norm<8>(a, s); break;
      }
    }
    // MXFP4 with enough rows to fill the CUs: four rows per wavefront where a
    // row fits eight wavefronts (K <= 4096), else two (K <= 8192), else one:
    // wider row groups load more rows per wavefront and write the
    // k-step-major arrays in longer runs (qkv shape: 12% fewer bytes written
    // to HBM, 2-3% less time with X read from HBM, 12% with X in cache).
    // Few rows (decode) keep one row per group, so that there
    // are more workgroups; NVFP4 too: its arithmetic, not its memory traffic,
    // sets its time, and fewer, larger workgroups were slower.
    if (FMT == 0 && a.m <= 32 && nblk <= 256 && !a.add) {
      // few rows: four lanes a block, one workgroup a row
      const int64_t w = (nblk * 4 + 63) / 64;
      const dim3 g((unsigned)a.m);
      if (w <= 1) prep_norm_quad_kernel<1><<<g, dim3(64), 0, s>>>(a);
      else if (w <= 2) prep_norm_quad_kernel<2><<<g, dim3(128), 0, s>>>(a);
      else if (w <= 4) prep_norm_quad_kernel<4><<<g, dim3(256), 0, s>>>(a);
      else if (w <= 8) prep_norm_quad_kernel<8><<<g, dim3(512), 0, s>>>(a);
      else prep_norm_quad_kernel<16><<<g, dim3(1024), 0, s>>>(a);
    } else if (FMT == 0 && a.m >= 1024 && nblk <= 8 * 16) launch_norm_rows<FMT, 4>(a, nblk, s);
    else if (FMT == 0 && a.m >= 512 && nblk <= 8 * 32) launch_norm_rows<FMT, 2>(a, nblk, s);
    else launch_norm_rows<FMT, 1>(a, nblk, s);
  } else {
    if (FMT == 1) {
      const int64_t total = a.m * nblk;
      const dim3 flat_grid((unsigned)((total + 255) / 256));
      amax_flat_kernel<<<dim3(min(flat_grid.x, kAmaxGrid)), 256, 0, s>>>(a.x, a.ld_x, a.m, a.k, a.amax);
    }
    if (ksm) {
      const uint32_t chunks = (uint32_t)((nblk + 3) / 4);
      const uint64_t waves = (uint64_t)((a.m + 15) / 16) * chunks;
      prep_flat_kernel<FMT, 16><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, s>>>(a, chunks);
    } else {
      const uint32_t chunks = (uint32_t)((nblk + 63) / 64);
      const uint64_t waves = (uint64_t)a.m * chunks;
      prep_flat_kernel<FMT, 1><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, s>>>(a, chunks);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- weights

// One lane per 32-element block of W: the same block quantizer as the
// residual of the preparation operator (no mask, no normalization).
template <int FMT>
__global__ __launch_bounds__(256) void quant_weight_kernel(QuantArgs a) {
  const int64_t nblk = a.k / 32;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.n * nblk) return;
  const int64_t row = gid / nblk, b = gid - row * nblk;
  uint32_t ww[16];
  float v[32];
  load32(a.w + row * a.ld_w + 32 * b, ww);
  unpack32(ww, v);
  uint32_t q[4], scales;
  if (FMT == 0) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, max(ww[i] & 0x7FFFu, (ww[i] >> 16) & 0x7FFFu));
    int ex = (int)(am >> 7);
    uint32_t sb = ex > 2 ? (uint32_t)(ex - 2) : 0u;
    float ss = e8m0_operand(sb);
    scales = sb;
    uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      bf16x2 pv = __builtin_bit_cast(bf16x2, ww[i]);
      uint32_t &x = w4[i >> 2];
      switch (i & 3) {
        case 0: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(x, pv, ss, 0); break;
        case 1: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(x, pv, ss, 1); break;
        case 2: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(x, pv, ss, 2); break;
        default: x = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(x, pv, ss, 3); break;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = w4[j];
  } else {
    float s_t = nv_tensor_scale(a.tensor_scale + 1);
    if (gid == 0) a.tensor_scale[0] = s_t;
    uint32_t a0 = 0, a1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) a0 = max(a0, max(ww[i] & 0x7FFFu, (ww[i] >> 16) & 0x7FFFu));
#pragma unroll
    for (int i = 8; i < 16; ++i) a1 = max(a1, max(ww[i] & 0x7FFFu, (ww[i] >> 16) & 0x7FFFu));
    float S[2];
    uint32_t sb0 = nv_scale(__uint_as_float(a0 << 16), s_t, S[0]);
    uint32_t sb1 = nv_scale(__uint_as_float(a1 << 16), s_t, S[1]);
    scales = sb0 | (sb1 << 8);
    nv_codes(v, S, q);
  }
  *reinterpret_cast<uint4 *>(a.codes + arr_off(row, b >> 2, a.ld_c, a.ksm, 64) + 16 * (b & 3)) =
      make_uint4(q[0], q[1], q[2], q[3]);
  store_scale<FMT, false>(a.scales, a.ld_s, a.ksm, row, b, scales);
}

template <int FMT>
hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
  const int64_t total = a.n * (a.k / 32);
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (FMT == 1) {
    zero_amax_kernel<<<1, 1, 0, s>>>(a.tensor_scale + 1);
    amax_flat_kernel<<<dim3(min(grid.x, kAmaxGrid)), block, 0, s>>>(a.w, a.ld_w, a.n, a.k, a.tensor_scale + 1);
  }
  quant_weight_kernel<FMT><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare_mx(const PrepArgs &a, hipStream_t s) { return launch_prepare<0>(a, s); }

hipError_t launch_prepare_silu_mx(const PrepArgs &a, hipStream_t s) {
  const int64_t nblk = a.k / 32;
  if (a.s_ksm) {
    const uint32_t chunks = (uint32_t)((nblk + 3) / 4);
    const uint64_t waves = (uint64_t)((a.m + 15) / 16) * chunks;
    prep_silu_kernel<16><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, s>>>(a, chunks);
  } else {
    const uint32_t chunks = (uint32_t)((nblk + 63) / 64);
    const uint64_t waves = (uint64_t)a.m * chunks;
    prep_silu_kernel<1><<<dim3((unsigned)((waves + 3) / 4)), 256, 0, s>>>(a, chunks);
  }
  return hipGetLastError();
}
hipError_t launch_prepare_nv(const PrepArgs &a, hipStream_t s) { return launch_prepare<1>(a, s); }

// ---------------------------------------------------------------- allocation-free entry point

// The workspace of sharq_prepare_noalloc: the NVFP4 tensor amax is reduced
// here instead of in the caller's tensor_scale[1].  Each GPU holds its own
// copy until the process ends; the host takes its address once per device
// (hipGetSymbolAddress with the device current) and passes that address to
// the kernels.  Every call on a GPU shares it (calls that overlap on one GPU
// race); each call clears it with a kernel before the amax passes.
constexpr int kNoallocScratchFloats = 64;   // 256 bytes; one float is used
static __device__ __align__(256) float scratch[kNoallocScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t launch_prepare_noalloc(PrepArgs a, int fmt, hipStream_t s) {
  if (fmt == 0) return launch_prepare<0>(a, s);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float *ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      e = hipGetSymbolAddress(reinterpret_cast<void **>(&g_scratch_ptr[dev]), HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch_ptr[dev] = nullptr;
        return e;
      }
    }
    ptr = g_scratch_ptr[dev];
  }
  a.amax = ptr;
  return launch_prepare<1>(a, s);
}
hipError_t launch_quantize_weight_mx(const QuantArgs &a, hipStream_t s) { return launch_quant<0>(a, s); }
hipError_t launch_quantize_weight_nv(const QuantArgs &a, hipStream_t s) { return launch_quant<1>(a, s); }

}  // namespace sharq
