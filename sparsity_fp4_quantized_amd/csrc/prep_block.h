// Per-block steps of the MXFP4 preparation, shared by the preparation
// kernels and by the GEMM whose epilogue prepares the down projection's input
// (SiLU(gate) * up formed from the gate+up accumulators).
//
// "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
// Inference" (arXiv:2606.26587), abstract, sentence 3: per block of 32 k of
// one row, the 2:4 magnitude mask, the FP4 backbone and the residual against
// the QUANTIZED backbone, each with its E8M0 block scale.
#pragma once

#include "fp4_device.h"
#include "kernels.h"

namespace sharq {

__device__ __forceinline__ void unpack32(const uint32_t w[16], float f[32]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

// E8M0 byte as the fp32 scale operand of the conversion instructions.
__device__ __forceinline__ float e8m0_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// ---------------------------------------------------------------- 2:4 mask

// Median of three unsigned values: one v_med3_u32 (the compiler does not form
// it from min/max on its own)
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Per group of four: keys order by magnitude, then by lower index.  u values
// are 3 - index of the two kept entries (umax for the lower index).
struct MaskOut {
  uint32_t top[8];        // largest key per group (for the block amax)
  uint32_t umax[8], umin[8];
  uint32_t meta;          // 8 nibbles i0 | i1 << 2
};

__device__ __forceinline__ void mask_block(const float xf[32], MaskOut &o) {
  uint32_t acc = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t k0 = (__float_as_uint(xf[4 * g + 0]) & 0x7FFF0000u) | 3u;
    uint32_t k1 = (__float_as_uint(xf[4 * g + 1]) & 0x7FFF0000u) | 2u;
    uint32_t k2 = (__float_as_uint(xf[4 * g + 2]) & 0x7FFF0000u) | 1u;
    uint32_t k3 = (__float_as_uint(xf[4 * g + 3]) & 0x7FFF0000u);
    // the largest and the median of k0..k2 (v_max3, v_med3), then k3 against
    // them: top = max(t3, k3), second = max(med, min(t3, k3))
    uint32_t t3 = max(max(k0, k1), k2);
    uint32_t md = med3_u32(k0, k1, k2);
    uint32_t top = max(t3, k3);
    uint32_t second = max(md, min(t3, k3));
    uint32_t ut = top & 3u, us = second & 3u;
    uint32_t umax = max(ut, us), umin = min(ut, us);
    o.top[g] = top;
    o.umax[g] = umax;
    o.umin[g] = umin;
    // nibble = (3 - umax) | (3 - umin) << 2 = 15 - (umax + 4 umin)
    acc |= (umax + (umin << 2)) << (4 * g);
  }
  o.meta = ~acc;
}

// ---------------------------------------------------------------- MXFP4 block

struct BlockOut {
  uint32_t meta;
  uint32_t s_comp[2];     // 8 compressed backbone bytes
  uint32_t s_dense[4];    // 32 backbone codes, dense layout
  uint32_t r_codes[4];    // 32 residual codes
  uint32_t s_scale, r_scale;
};

// xw: the 32 normalized values as bf16 pairs; xf: the same values as fp32.
__device__ __forceinline__ void quantize_block_mx(const uint32_t xw[16], const float xf[32],
                                                  BlockOut &o) {
  MaskOut mk;
  mask_block(xf, mk);
  o.meta = mk.meta;

  // backbone scale: each group keeps its largest entry, so the backbone's
  // block amax is the block amax of x_n
  uint32_t am = 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) am = max(am, mk.top[g]);
  int ex = (int)(am >> 23);
  uint32_t sb = ex > 2 ? (uint32_t)(ex - 2) : 0u;
  float ss = e8m0_operand(sb);
  o.s_scale = sb;

  // compressed backbone: v_perm gathers (x[i0], x[i1]) as a bf16 pair, one
  // conversion gives the byte (code at i0 low, code at i1 high)
  uint32_t comp[2] = {0u, 0u};
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t z = mk.umax[g] | (mk.umin[g] << 16);
    // selector bytes 2 i0, 2 i0 + 1, 2 i1, 2 i1 + 1 (z < 2^18: a 24-bit multiply)
    uint32_t sel = 0x07060706u - __umul24(z, 0x0202u);
    uint32_t pair = __builtin_amdgcn_perm(xw[2 * g + 1], xw[2 * g], sel);
    bf16x2 pv = __builtin_bit_cast(bf16x2, pair);
    uint32_t &w = comp[g >> 2];
    switch (g & 3) {
      case 0: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 0); break;
      case 1: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 1); break;
      case 2: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 2); break;
      default: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 3); break;
    }
  }
  o.s_comp[0] = comp[0];
  o.s_comp[1] = comp[1];

  // dense backbone codes: all codes, then the dropped nibbles cleared
  uint32_t full[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    bf16x2 pv = __builtin_bit_cast(bf16x2, xw[i]);
    uint32_t &w = full[i >> 2];
    switch (i & 3) {
      case 0: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 0); break;
      case 1: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 1); break;
      case 2: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 2); break;
      default: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, pv, ss, 3); break;
    }
  }
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

  // residual against the quantized backbone (exact in fp32)
  float res[32];
  float ramax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f32x2 d;
    switch (i & 3) {
      case 0: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], ss, 0); break;
      case 1: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], ss, 1); break;
      case 2: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], ss, 2); break;
      default: d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(o.s_dense[i >> 2], ss, 3); break;
    }
    res[2 * i] = xf[2 * i] - d[0];
    res[2 * i + 1] = xf[2 * i + 1] - d[1];
    ramax = fmaxf(fmaxf(ramax, fabsf(res[2 * i])), fabsf(res[2 * i + 1]));
  }
  int rex = (int)(__float_as_uint(ramax) >> 23);
  uint32_t rb = rex > 2 ? (uint32_t)(rex - 2) : 0u;
  float rs = e8m0_operand(rb);
  o.r_scale = rb;
  uint32_t rc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t &w = rc[i >> 2];
    switch (i & 3) {
      case 0: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, res[2 * i], res[2 * i + 1], rs, 0); break;
      case 1: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, res[2 * i], res[2 * i + 1], rs, 1); break;
      case 2: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, res[2 * i], res[2 * i + 1], rs, 2); break;
      default: w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, res[2 * i], res[2 * i + 1], rs, 3); break;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) o.r_codes[q] = rc[q];
}

// Stores of the lane's 32 k (block b of row `row`): every array of a view in
// its layout (arr_off: row-major, or k-step-major with 4 blocks of 32 k per
// 128-k step).  Scales: MXFP4 one byte, NVFP4 two.
//
// NT: non-temporal stores, for kernels whose wavefronts write whole 128-byte
// lines (four or sixteen rows of a k-step, or 64 blocks of one row).  The GEMM
// that reads these arrays runs after this kernel and mostly on other XCDs, so
// kept in this XCD's L2 they are only dirty lines to write back at the
// kernel's end (measured: down_prefill 21.9 -> 17.3 us, qkv_prefill -3%).
// With one row per wavefront a store of the k-step-major arrays writes
// sixteen pieces of 2-32 bytes, and non-temporal partial lines made the
// NVFP4 preparation 40% slower: those kernels store normally.
template <bool NT, class T>
__device__ __forceinline__ void put(T v, T *p) {
  if (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int FMT, bool NT>
__device__ __forceinline__ void store_scale(uint8_t *base, int64_t ld, int ksm, int64_t row,
                                            int64_t b, uint32_t v) {
  if (FMT == 0) {
    put<NT>((uint8_t)v, base + arr_off(row, b >> 2, ld, ksm, 4) + (b & 3));
  } else {
    put<NT>((uint16_t)v, reinterpret_cast<uint16_t *>(base + arr_off(row, b >> 2, ld, ksm, 8) + 2 * (b & 3)));
  }
}

template <int FMT, bool NT>
__device__ __forceinline__ void store_block(const PrepArgs &a, int64_t row, int64_t b,
                                            const BlockOut &o) {
  const int64_t t = b >> 2, q = b & 3;
  put<NT>(u32x2{o.s_comp[0], o.s_comp[1]},
          reinterpret_cast<u32x2 *>(a.s_codes + arr_off(row, t, a.ld_sc, a.s_ksm, 32) + 8 * q));
  put<NT>(o.meta, reinterpret_cast<uint32_t *>(a.meta + arr_off(row, t, a.ld_meta, a.s_ksm, 16) + 4 * q));
  put<NT>(u32x4{o.r_codes[0], o.r_codes[1], o.r_codes[2], o.r_codes[3]},
          reinterpret_cast<u32x4 *>(a.r_codes + arr_off(row, t, a.ld_rc, a.r_ksm, 64) + 16 * q));
  if (a.s_dense)
    put<NT>(u32x4{o.s_dense[0], o.s_dense[1], o.s_dense[2], o.s_dense[3]},
            reinterpret_cast<u32x4 *>(a.s_dense + arr_off(row, t, a.ld_sd, a.s_ksm, 64) + 16 * q));
  store_scale<FMT, NT>(a.s_scales, a.ld_ss, a.s_ksm, row, b, o.s_scale);
  store_scale<FMT, NT>(a.r_scales, a.ld_rs, a.r_ksm, row, b, o.r_scale);
}

// arr_off is linear in the row and the k-step, so the offset of (rs + rl,
// ts + tl) splits into arr_off(rs, ts), wavefront-uniform (64-bit, scalar
// registers), plus this lane part.  Every array of a view spans less than
// 4 GiB, so the lane part fits 32 bits and the store takes a scalar base and a
// 32-bit vector offset.
template <int BPS>
__device__ __forceinline__ uint32_t lane_off(int64_t ld, int ksm, uint32_t rl, uint32_t tl) {
  return ksm ? tl * ((uint32_t)ld * BPS) + rl * BPS : rl * (uint32_t)ld + tl * BPS;
}

// The lane parts of one lane's block in every array of a view pair: row rl of
// the row group, k-step tl of the pass, block q of the k-step.
struct LaneOffsets {
  uint32_t sc, meta, rc, sd, ss, rs;
};

template <int FMT>
__device__ __forceinline__ LaneOffsets lane_offsets(const PrepArgs &a, uint32_t rl, uint32_t tl,
                                                    uint32_t q) {
  constexpr int SB = FMT == 0 ? 4 : 8;   // scale bytes per row and k-step
  LaneOffsets o;
  o.sc = lane_off<32>(a.ld_sc, a.s_ksm, rl, tl) + 8 * q;
  o.meta = lane_off<16>(a.ld_meta, a.s_ksm, rl, tl) + 4 * q;
  o.rc = lane_off<64>(a.ld_rc, a.r_ksm, rl, tl) + 16 * q;
  o.sd = a.s_dense ? lane_off<64>(a.ld_sd, a.s_ksm, rl, tl) + 16 * q : 0u;
  o.ss = lane_off<SB>(a.ld_ss, a.s_ksm, rl, tl) + (SB / 4) * q;
  o.rs = lane_off<SB>(a.ld_rs, a.r_ksm, rl, tl) + (SB / 4) * q;
  return o;
}

// store_block for the block at row rs + rl, k-step ts + tl, given the uniform
// (rs, ts) and the lane parts.
template <int FMT, bool NT>
__device__ __forceinline__ void store_block_at(const PrepArgs &a, int64_t rs, int64_t ts,
                                               const LaneOffsets &lo, const BlockOut &o) {
  constexpr int SB = FMT == 0 ? 4 : 8;
  put<NT>(u32x2{o.s_comp[0], o.s_comp[1]},
          reinterpret_cast<u32x2 *>(a.s_codes + arr_off(rs, ts, a.ld_sc, a.s_ksm, 32) + lo.sc));
  put<NT>(o.meta, reinterpret_cast<uint32_t *>(a.meta + arr_off(rs, ts, a.ld_meta, a.s_ksm, 16) + lo.meta));
  put<NT>(u32x4{o.r_codes[0], o.r_codes[1], o.r_codes[2], o.r_codes[3]},
          reinterpret_cast<u32x4 *>(a.r_codes + arr_off(rs, ts, a.ld_rc, a.r_ksm, 64) + lo.rc));
  if (a.s_dense)
    put<NT>(u32x4{o.s_dense[0], o.s_dense[1], o.s_dense[2], o.s_dense[3]},
            reinterpret_cast<u32x4 *>(a.s_dense + arr_off(rs, ts, a.ld_sd, a.s_ksm, 64) + lo.sd));
  uint8_t *ps = a.s_scales + arr_off(rs, ts, a.ld_ss, a.s_ksm, SB) + lo.ss;
  uint8_t *pr = a.r_scales + arr_off(rs, ts, a.ld_rs, a.r_ksm, SB) + lo.rs;
  if (FMT == 0) {
    put<NT>((uint8_t)o.s_scale, ps);
    put<NT>((uint8_t)o.r_scale, pr);
  } else {
    put<NT>((uint16_t)o.s_scale, reinterpret_cast<uint16_t *>(ps));
    put<NT>((uint16_t)o.r_scale, reinterpret_cast<uint16_t *>(pr));
  }
}

// fl32(v / S) from y = fl32(1 / S): q0 = fl32(v y) is within an ulp of v / S,
// r = fma(-q0, S, v) is then exact, and fma(r, y, q0) is the correctly rounded
// quotient (Markstein's correction of a faithful quotient with a correctly
// rounded reciprocal).  Valid while neither y nor the quotient nor the
// remainder leaves the normal range: the NVFP4 scales S in [2^-100, 2^100]
// with |v / S| < 8, and the row mean below.  Host and device: a host build
// checks it against IEEE division over the row mean's whole domain.
__host__ __device__ __forceinline__ float div_rn(float v, float S, float y) {
  const float q0 = v * y;
  const float r = __builtin_fmaf(-q0, S, v);
  return __builtin_fmaf(r, y, q0);
}

// The row mean fl32(ss / k) for k = 32 .. 16384 from inv_k = fl32(1 / k):
// Markstein's correction where no step can leave the normal range (ss = 0 or
// ss in [2^-100, 2^100]), an IEEE division otherwise (zero rows aside,
// practically never: ss is a sum of squares of bf16 values).
__host__ __device__ __forceinline__ float row_mean_of(float ss, float kf, float inv_k) {
  if (ss == 0.0f || (ss >= 0x1p-100f && ss <= 0x1p100f)) return div_rn(ss, kf, inv_k);
  return ss / kf;
}

// SiLU(gate) * up in front of the down projection: x = bf16 of g / (1 +
// exp(-g)) * u evaluated in binary64 and rounded once.  The lane evaluates
// it in fp32 first and keeps that when rounding it must give the same bf16
// as the exact value: when v's bits are more than 64 units in the last place
// away from a bf16 rounding midpoint (low half 0x8000) and v is within fewer
// than 64 units of the exact value.  Otherwise (about 1 in 500, and for |g|
// outside [2^-60, 8]) the lane evaluates in binary64 and rounds that:
// directly to 8 significant bits, ties to even, for |v| >= 2^-126, through
// float below.  A double exp differs from another correctly implemented one
// by at most an ulp, so only a value within 2^-51 of a midpoint could round
// differently.
// The rounding itself is IEEE nearest-even with overflow: |v| >= 2^128 (or a
// carry out of the largest binade) gives Inf, a NaN gives a quiet NaN of the
// same sign.  Host and device: a host build of this header checks it against
// the CPU reference on every branch.
__host__ __device__ __forceinline__ uint32_t bf16_of_double(double v) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, v);
  const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
  const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
  if (mag > 0x7FF0000000000000ull) return sign | 0x7FC0u;   // NaN
  if (mag >= (1151ull << 52)) return sign | 0x7F80u;        // |v| >= 2^128, Inf
  if (mag < (897ull << 52)) {                               // |v| < 2^-126
    const uint32_t f = __builtin_bit_cast(uint32_t, (float)v);
    return (f + 0x7FFFu + ((f >> 16) & 1u)) >> 16;
  }
  // exponent | 7 bits, nearest even; a carry out of the 2^127 binade lands
  // on exactly 0x7F80 (Inf)
  const uint64_t r = (mag + 0xFFFFFFFFFFFull + ((mag >> 45) & 1ull)) >> 45;
  return sign | (uint32_t)(r - ((uint64_t)(1023 - 127) << 7));
}

// The fp32 evaluation: true, with its bf16 rounding in x, when that is the
// exact value's bf16.  It uses the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32, each within 1 ulp): t = -g log2(e) carries two fp32
// roundings, so e = 2^t is within (|g| + 1) 2^-23 of exp(-g) relatively, and
// with 1 + e, the reciprocal and the two products v is within (|g| + 3.5)
// 2^-23 of the exact value, at most 23 units in its last place for
// |g| <= 8: well inside the 64-unit guard.  (The exactly rounded expf and
// IEEE division took about 36 instructions a value; this takes about 15.)
// No branch, so that a lane can evaluate many values at once and repeat
// only the few that need it in binary64.
__device__ __forceinline__ bool silu_mul_fast(float g, float u, uint32_t &x) {
  const float ag = __builtin_fabsf(g);
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504f);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  const float sg = g * r;
  const float v = sg * u;
  const uint32_t b = __float_as_uint(v);
  const int off = (int)(b & 0xFFFFu) - 0x8000;
  x = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return ag >= 0x1p-60f && ag <= 8.0f && (off > 64 || off < -64);
}

// The binary64 evaluation, rounded once to bf16.
__device__ __forceinline__ uint32_t silu_mul_slow(float g, float u) {
  const double gd = (double)g, ud = (double)u;
  const double sd = gd / (1.0 + exp(-gd));
  return bf16_of_double(sd * ud);
}

__device__ __forceinline__ uint32_t silu_mul_bf16(float g, float u) {
  uint32_t x;
  return silu_mul_fast(g, u, x) ? x : silu_mul_slow(g, u);
}

}  // namespace sharq
