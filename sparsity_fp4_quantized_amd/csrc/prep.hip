// Fused preparation operator of the SharQ path, for gfx950.
//
// "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
// Inference" (arXiv:2606.26587), abstract, sentence 3 (input-adaptive N:M
// mask, FP4 backbone, residual against the quantized backbone) and sentence 5
// (one fused operator that also absorbs the layer normalization).
//
// One wavefront owns one row of X.  Lane l owns the 32-element K blocks
// b = c * 64 + l (c = 0, 1, ...), so each lane reads 64 contiguous bytes per
// block and a block's MX scale, its eight 2:4 groups and all its output bytes
// stay inside one lane.  The RMS reduction follows a fixed binary tree: a
// tree over the 32 squares inside the lane, a xor butterfly across the 64
// lanes (the 2048-element chunk sums) and a tree over the chunks, which is the
// pairwise tree over 2^ceil(log2 K) leaves.  With normalization the row stays
// in registers between the reduction and the quantization (one HBM pass).
#include "fp4_device.h"
#include "kernels.h"

namespace sharq {
namespace {

constexpr int kRowsPerBlock = 4;   // four wavefronts, one row each

struct Block32 {
  uint32_t v[16];   // 32 bf16, element 2i in the low half of v[i]
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// X is read exactly once: non-temporal loads keep it from displacing the
// outputs and the next kernel's operands in the caches.
__device__ __forceinline__ void load_block(const uint16_t *p, Block32 &b) {
  const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    u32x4 t = __builtin_nontemporal_load(q + i);
    b.v[4 * i + 0] = t.x;
    b.v[4 * i + 1] = t.y;
    b.v[4 * i + 2] = t.z;
    b.v[4 * i + 3] = t.w;
  }
}

// Tree sum of the 32 squares of a block (adjacent pairs at every level).
__device__ __forceinline__ float block_sumsq(const Block32 &b) {
  float q[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float lo = bf16_lo(b.v[i]), hi = bf16_hi(b.v[i]);
    q[2 * i] = lo * lo;
    q[2 * i + 1] = hi * hi;
  }
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) q[i] = q[2 * i] + q[2 * i + 1];
  }
  return q[0];
}

__device__ __forceinline__ float wave_tree_sum(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = v + __shfl_xor(v, off, 64);
  return v;
}

// x_n = bf16((x * r) * gamma) for the 32 elements of a block.
__device__ __forceinline__ void normalize_block(Block32 &b, const uint16_t *g, float r) {
  Block32 gb;
  const uint4 *q = reinterpret_cast<const uint4 *>(g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 t = q[i];
    gb.v[4 * i + 0] = t.x;
    gb.v[4 * i + 1] = t.y;
    gb.v[4 * i + 2] = t.z;
    gb.v[4 * i + 3] = t.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float lo = (bf16_lo(b.v[i]) * r) * bf16_lo(gb.v[i]);
    float hi = (bf16_hi(b.v[i]) * r) * bf16_hi(gb.v[i]);
    b.v[i] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
  }
}

// 2:4 mask of one group from 15-bit magnitudes: keep the two largest, lower
// index first on ties.  Returns the 4-bit keep mask and the meta nibble.
__device__ __forceinline__ void mask_group(const uint32_t mag[4], uint32_t &keep,
                                           uint32_t &nibble) {
  // unique keys: magnitude, then lower index ranks higher
  uint32_t k0 = (mag[0] << 2) | 3u, k1 = (mag[1] << 2) | 2u;
  uint32_t k2 = (mag[2] << 2) | 1u, k3 = (mag[3] << 2) | 0u;
  uint32_t a = max(k0, k1), b = min(k0, k1), c = max(k2, k3), d = min(k2, k3);
  uint32_t top = max(a, c);
  uint32_t second = max(min(a, c), max(b, d));
  keep = (k0 >= second ? 1u : 0u) | (k1 >= second ? 2u : 0u) | (k2 >= second ? 4u : 0u) |
         (k3 >= second ? 8u : 0u);
  uint32_t it = 3u - (top & 3u), is = 3u - (second & 3u);
  uint32_t i0 = min(it, is), i1 = max(it, is);
  nibble = i0 | (i1 << 2);
  (void)top;
}

struct BlockOut {
  uint32_t meta;        // 8 nibbles
  uint32_t s_comp[2];   // 8 compressed bytes
  uint32_t s_dense[4];  // 32 dense codes
  uint32_t r_codes[4];  // 32 dense codes
  uint32_t s_scale;     // MX: 1 byte; NV: 2 bytes
  uint32_t r_scale;
};

// Compressed backbone byte of a group: code at i0 low, code at i1 high.
__device__ __forceinline__ uint32_t compress_group(uint32_t dense16, uint32_t nibble) {
  uint32_t i0 = nibble & 3u, i1 = nibble >> 2;
  uint32_t c0 = (dense16 >> (4u * i0)) & 15u;
  uint32_t c1 = (dense16 >> (4u * i1)) & 15u;
  return c0 | (c1 << 4);
}

// FMT 0: MXFP4 (one 32-block); FMT 1: NVFP4 (two 16-blocks, tensor scale s_t).
template <int FMT>
__device__ __forceinline__ void quantize_block(const Block32 &xn, float s_t, BlockOut &o) {
  uint32_t mag[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    mag[2 * i] = xn.v[i] & 0x7FFFu;
    mag[2 * i + 1] = (xn.v[i] >> 16) & 0x7FFFu;
  }
  uint32_t keep = 0;
  o.meta = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t kg, nib;
    mask_group(&mag[4 * g], kg, nib);
    keep |= kg << (4 * g);
    o.meta |= nib << (4 * g);
  }

  float xf[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    xf[2 * i] = bf16_lo(xn.v[i]);
    xf[2 * i + 1] = bf16_hi(xn.v[i]);
  }

  uint32_t sc[32], rc[32];
  float res[32];
  constexpr int kBlk = FMT == 0 ? 32 : 16;
  o.s_scale = 0;
  o.r_scale = 0;
#pragma unroll
  for (int h = 0; h < 32 / kBlk; ++h) {
    // backbone: block amax of x_n equals that of the kept values
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < kBlk; ++i) am = max(am, mag[h * kBlk + i]);
    if (FMT == 0) {
      uint32_t sb = e8m0_from_amax_bits(am << 16);
      float inv = e8m0_inv(sb), val = e8m0_val(sb);
      o.s_scale |= sb << (8 * h);
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        int j = h * kBlk + i;
        bool kp = (keep >> j) & 1u;
        uint32_t c = kp ? e2m1_encode(xf[j] * inv) : 0u;
        float d = kp ? e2m1_value(c) * val : 0.0f;
        sc[j] = c;
        res[j] = xf[j] - d;
      }
    } else {
      float d6 = 6.0f * s_t;
      float ratio = __uint_as_float(am << 16) / d6;
      uint32_t sb = e4m3_encode_pos(ratio);
      float S = e4m3_value(sb) * s_t;
      o.s_scale |= sb << (8 * h);
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        int j = h * kBlk + i;
        bool kp = (keep >> j) & 1u;
        uint32_t c;
        float d;
        if (S == 0.0f) {
          c = (__float_as_uint(xf[j]) >> 28) & 8u;
          d = __uint_as_float((c & 8u) << 28);
        } else {
          c = e2m1_encode(xf[j] / S);
          d = e2m1_value(c) * S;
        }
        c = kp ? c : 0u;
        d = kp ? d : 0.0f;
        sc[j] = c;
        res[j] = xf[j] - d;
      }
    }
    // residual
    uint32_t ar = 0;
#pragma unroll
    for (int i = 0; i < kBlk; ++i) ar = max(ar, __float_as_uint(res[h * kBlk + i]) & 0x7FFFFFFFu);
    if (FMT == 0) {
      uint32_t rb = e8m0_from_amax_bits(ar);
      float inv = e8m0_inv(rb);
      o.r_scale |= rb << (8 * h);
#pragma unroll
      for (int i = 0; i < kBlk; ++i) rc[h * kBlk + i] = e2m1_encode(res[h * kBlk + i] * inv);
    } else {
      float d6 = 6.0f * s_t;
      float ratio = __uint_as_float(ar) / d6;
      uint32_t rb = e4m3_encode_pos(ratio);
      float S = e4m3_value(rb) * s_t;
      o.r_scale |= rb << (8 * h);
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        float v = res[h * kBlk + i];
        rc[h * kBlk + i] = (S == 0.0f) ? ((__float_as_uint(v) >> 28) & 8u) : e2m1_encode(v / S);
      }
    }
  }

#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t s = 0, r = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s |= sc[8 * q + i] << (4 * i);
      r |= rc[8 * q + i] << (4 * i);
    }
    o.s_dense[q] = s;
    o.r_codes[q] = r;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t w = 0;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      int g = 4 * q + gg;
      uint32_t dense16 = (o.s_dense[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
      w |= compress_group(dense16, (o.meta >> (4 * g)) & 15u) << (8 * gg);
    }
    o.s_comp[q] = w;
  }
}

template <int FMT>
__device__ __forceinline__ void store_block(const PrepArgs &a, int64_t row, int b,
                                            const BlockOut &o) {
  *reinterpret_cast<uint2 *>(a.s_codes + row * a.ld_sc + 8 * b) = make_uint2(o.s_comp[0], o.s_comp[1]);
  *reinterpret_cast<uint32_t *>(a.meta + row * a.ld_meta + 4 * b) = o.meta;
  *reinterpret_cast<uint4 *>(a.r_codes + row * a.ld_rc + 16 * b) =
      make_uint4(o.r_codes[0], o.r_codes[1], o.r_codes[2], o.r_codes[3]);
  if (a.s_dense)
    *reinterpret_cast<uint4 *>(a.s_dense + row * a.ld_sd + 16 * b) =
        make_uint4(o.s_dense[0], o.s_dense[1], o.s_dense[2], o.s_dense[3]);
  if (FMT == 0) {
    a.s_scales[row * a.ld_ss + b] = (uint8_t)o.s_scale;
    a.r_scales[row * a.ld_rs + b] = (uint8_t)o.r_scale;
  } else {
    *reinterpret_cast<uint16_t *>(a.s_scales + row * a.ld_ss + 2 * b) = (uint16_t)o.s_scale;
    *reinterpret_cast<uint16_t *>(a.r_scales + row * a.ld_rs + 2 * b) = (uint16_t)o.r_scale;
  }
}

__device__ __forceinline__ float nv_tensor_scale(const float *ts) {
  float amax = ts[1];
  return amax == 0.0f ? 1.0f : amax / 2688.0f;
}

// Row RMS scale r = 1 / sqrt(ss / k + eps) from the row held in registers.
template <int NB>
__device__ __forceinline__ float row_rms_scale(const Block32 (&xb)[NB], int lane, int nblk,
                                               int64_t k, float eps) {
  float cs[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    float s = (c * 64 + lane < nblk) ? block_sumsq(xb[c]) : 0.0f;
    cs[c] = wave_tree_sum(s);
  }
#pragma unroll
  for (int w = NB / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w; ++i) cs[i] = cs[2 * i] + cs[2 * i + 1];
  }
  float mean = cs[0] / (float)k;
  float var = mean + eps;
  float s = __builtin_sqrtf(var);
  return 1.0f / s;
}

template <int FMT, int NB>
__global__ __launch_bounds__(256) void prep_norm_kernel(PrepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.m) return;
  const int nblk = (int)(a.k / 32);
  const uint16_t *xr = a.x + row * a.ld_x;
  Block32 xb[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    int b = c * 64 + lane;
    if (b < nblk) load_block(xr + 32 * b, xb[c]);
  }
  float r = row_rms_scale<NB>(xb, lane, nblk, a.k, a.eps);
  float s_t = FMT == 1 ? nv_tensor_scale(a.tensor_scale) : 1.0f;
  if (FMT == 1 && row == 0 && lane == 0) a.tensor_scale[0] = s_t;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    int b = c * 64 + lane;
    if (b < nblk) {
      normalize_block(xb[c], a.gamma + 32 * b, r);
      BlockOut o;
      quantize_block<FMT>(xb[c], s_t, o);
      store_block<FMT>(a, row, b, o);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void prep_plain_kernel(PrepArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.m) return;
  const int nblk = (int)(a.k / 32);
  const uint16_t *xr = a.x + row * a.ld_x;
  float s_t = FMT == 1 ? nv_tensor_scale(a.tensor_scale) : 1.0f;
  if (FMT == 1 && row == 0 && lane == 0) a.tensor_scale[0] = s_t;
  for (int b = lane; b < nblk; b += 64) {
    Block32 xb;
    load_block(xr + 32 * b, xb);
    BlockOut o;
    quantize_block<FMT>(xb, s_t, o);
    store_block<FMT>(a, row, b, o);
  }
}

// NVFP4 tensor amax of x_n: reduce |x_n| over the row, one atomic max per wave
// (fp32 bit patterns of non-negative values order like unsigned integers).
template <int NB, bool NORM>
__global__ __launch_bounds__(256) void amax_rows_kernel(const uint16_t *x, int64_t ld_x,
                                                        int64_t m, int64_t k,
                                                        const uint16_t *gamma, float eps,
                                                        float *ts) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= m) return;
  const int nblk = (int)(k / 32);
  const uint16_t *xr = x + row * ld_x;
  uint32_t am = 0;
  if (NORM) {
    Block32 xb[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      int b = c * 64 + lane;
      if (b < nblk) load_block(xr + 32 * b, xb[c]);
    }
    float r = row_rms_scale<NB>(xb, lane, nblk, k, eps);
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      int b = c * 64 + lane;
      if (b < nblk) {
        normalize_block(xb[c], gamma + 32 * b, r);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          am = max(am, max(xb[c].v[i] & 0x7FFFu, (xb[c].v[i] >> 16) & 0x7FFFu));
      }
    }
  } else {
    for (int b = lane; b < nblk; b += 64) {
      Block32 xb;
      load_block(xr + 32 * b, xb);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        am = max(am, max(xb.v[i] & 0x7FFFu, (xb.v[i] >> 16) & 0x7FFFu));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 64));
  if (lane == 0) atomicMax(reinterpret_cast<unsigned int *>(ts + 1), am << 16);
}

__global__ void zero_amax_kernel(float *ts) { ts[1] = 0.0f; }

int pick_nb(int64_t k) {
  int64_t chunks = (k / 32 + 63) / 64;
  int nb = 1;
  while (nb < chunks) nb <<= 1;
  return nb;
}

template <int FMT>
hipError_t launch_prepare(const PrepArgs &a, hipStream_t s) {
  dim3 grid((unsigned)((a.m + kRowsPerBlock - 1) / kRowsPerBlock)), block(256);
  if (FMT == 1) {
    zero_amax_kernel<<<1, 1, 0, s>>>(a.tensor_scale);
    if (a.gamma) {
      switch (pick_nb(a.k)) {
        case 1: amax_rows_kernel<1, true><<<grid, block, 0, s>>>(a.x, a.ld_x, a.m, a.k, a.gamma, a.eps, a.tensor_scale); break;
        case 2: amax_rows_kernel<2, true><<<grid, block, 0, s>>>(a.x, a.ld_x, a.m, a.k, a.gamma, a.eps, a.tensor_scale); break;
        case 4: amax_rows_kernel<4, true><<<grid, block, 0, s>>>(a.x, a.ld_x, a.m, a.k, a.gamma, a.eps, a.tensor_scale); break;
        default: amax_rows_kernel<8, true><<<grid, block, 0, s>>>(a.x, a.ld_x, a.m, a.k, a.gamma, a.eps, a.tensor_scale); break;
      }
    } else {
      amax_rows_kernel<1, false><<<grid, block, 0, s>>>(a.x, a.ld_x, a.m, a.k, nullptr, a.eps, a.tensor_scale);
    }
  }
  if (a.gamma) {
    switch (pick_nb(a.k)) {
      case 1: prep_norm_kernel<FMT, 1><<<grid, block, 0, s>>>(a); break;
      case 2: prep_norm_kernel<FMT, 2><<<grid, block, 0, s>>>(a); break;
      case 4: prep_norm_kernel<FMT, 4><<<grid, block, 0, s>>>(a); break;
      default: prep_norm_kernel<FMT, 8><<<grid, block, 0, s>>>(a); break;
    }
  } else {
    prep_plain_kernel<FMT><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- weights

// One lane per 32-element block of W (flat over rows); same block quantizer
// as the residual of the preparation operator.
template <int FMT>
__global__ __launch_bounds__(256) void quant_weight_kernel(QuantArgs a) {
  const int64_t nblk = a.k / 32;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.n * nblk) return;
  const int64_t row = gid / nblk;
  const int b = (int)(gid - row * nblk);
  Block32 wb;
  load_block(a.w + row * a.ld_w + 32 * b, wb);
  float s_t = 1.0f;
  if (FMT == 1) {
    s_t = nv_tensor_scale(a.tensor_scale);
    if (gid == 0) a.tensor_scale[0] = s_t;
  }
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = bf16_lo(wb.v[i]);
    v[2 * i + 1] = bf16_hi(wb.v[i]);
  }
  uint32_t c[32];
  uint32_t scales = 0;
  constexpr int kBlk = FMT == 0 ? 32 : 16;
#pragma unroll
  for (int h = 0; h < 32 / kBlk; ++h) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < kBlk; ++i) am = max(am, __float_as_uint(v[h * kBlk + i]) & 0x7FFFFFFFu);
    if (FMT == 0) {
      uint32_t sb = e8m0_from_amax_bits(am);
      float inv = e8m0_inv(sb);
      scales |= sb << (8 * h);
#pragma unroll
      for (int i = 0; i < kBlk; ++i) c[h * kBlk + i] = e2m1_encode(v[h * kBlk + i] * inv);
    } else {
      float ratio = __uint_as_float(am) / (6.0f * s_t);
      uint32_t sb = e4m3_encode_pos(ratio);
      float S = e4m3_value(sb) * s_t;
      scales |= sb << (8 * h);
#pragma unroll
      for (int i = 0; i < kBlk; ++i) {
        float t = v[h * kBlk + i];
        c[h * kBlk + i] = (S == 0.0f) ? ((__float_as_uint(t) >> 28) & 8u) : e2m1_encode(t / S);
      }
    }
  }
  uint32_t q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= c[8 * j + i] << (4 * i);
    q[j] = w;
  }
  *reinterpret_cast<uint4 *>(a.codes + row * a.ld_c + 16 * b) = make_uint4(q[0], q[1], q[2], q[3]);
  if (FMT == 0)
    a.scales[row * a.ld_s + b] = (uint8_t)scales;
  else
    *reinterpret_cast<uint16_t *>(a.scales + row * a.ld_s + 2 * b) = (uint16_t)scales;
}

__global__ __launch_bounds__(256) void amax_flat_kernel(const uint16_t *w, int64_t ld_w, int64_t n,
                                                        int64_t k, float *ts) {
  const int64_t nblk = k / 32;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t am = 0;
  if (gid < n * nblk) {
    const int64_t row = gid / nblk;
    const int b = (int)(gid - row * nblk);
    Block32 wb;
    load_block(w + row * ld_w + 32 * b, wb);
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, max(wb.v[i] & 0x7FFFu, (wb.v[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<unsigned int *>(ts + 1), am << 16);
}

template <int FMT>
hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
  const int64_t total = a.n * (a.k / 32);
  dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (FMT == 1) {
    zero_amax_kernel<<<1, 1, 0, s>>>(a.tensor_scale);
    amax_flat_kernel<<<grid, block, 0, s>>>(a.w, a.ld_w, a.n, a.k, a.tensor_scale);
  }
  quant_weight_kernel<FMT><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare_mx(const PrepArgs &a, hipStream_t s) { return launch_prepare<0>(a, s); }
hipError_t launch_prepare_nv(const PrepArgs &a, hipStream_t s) { return launch_prepare<1>(a, s); }
hipError_t launch_quantize_weight_mx(const QuantArgs &a, hipStream_t s) { return launch_quant<0>(a, s); }
hipError_t launch_quantize_weight_nv(const QuantArgs &a, hipStream_t s) { return launch_quant<1>(a, s); }

}  // namespace sharq
