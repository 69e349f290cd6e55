// Device-side FP4 / FP8 helpers for the gfx950 kernels.
//
// Value rules: E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and
// E8M0 scales (2^(byte-127)) from the OCP Microscaling v1.0 specification;
// E4M3 from the OCP 8-bit floating point specification.  Rounding is to
// nearest, ties to even, saturating; the sign of zero is kept.  These are the
// element and scale formats named in the SharQ abstract (arXiv:2606.26587,
// sentence 7: MXFP4 and NVFP4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {

// clang vector types (not HIP's uint4 struct), so that values stay in registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// E2M1 code (4 bits) of t: nearest magnitude, ties to even code, saturate at 6,
// sign bit = sign bit of t.  Exact for every finite fp32 t.
__device__ __forceinline__ uint32_t e2m1_encode(float t) {
  uint32_t u = __float_as_uint(t);
  uint32_t sign = (u >> 28) & 8u;
  uint32_t a = u & 0x7FFFFFFFu;
  // |t| < 1: codes 0, 1, 2 are rint(2|t|) with ties to even (0.25 -> 0, 0.75 -> 2)
  uint32_t small = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
  // |t| >= 1: round the fp32 pattern to one mantissa bit (nearest even); the
  // exponent/mantissa pair then counts codes from 1.0 (code 2) upward
  uint32_t r = (a + 0x1FFFFFu + ((a >> 22) & 1u)) >> 22;
  uint32_t big = r - 252u;
  big = big > 7u ? 7u : big;
  uint32_t m = (a < 0x3F800000u) ? small : big;
  return sign | m;
}

// Magnitude of an E2M1 code as fp32 (exact), sign applied.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  uint32_t m = code & 7u;
  // m >= 2: exponent (m >> 1) - 1, mantissa bit m & 1; m == 1: 0.5; m == 0: 0
  uint32_t bits = (m >= 2u) ? ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22))
                            : (m == 1u ? 0x3F000000u : 0u);
  return __uint_as_float(bits | ((code & 8u) << 28));
}

// E8M0 byte of the MX block scale for a block whose largest magnitude has the
// fp32 bit pattern amax_bits (sign cleared): floor(log2 amax) - 2 + 127,
// clamped at 0 (this also covers amax = 0 and subnormal amax).
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
  int ex = (int)(amax_bits >> 23);
  return ex > 2 ? (uint32_t)(ex - 2) : 0u;
}

// 2^(127 - byte) and 2^(byte - 127) as fp32 (exact; 2^-127 is subnormal).
__device__ __forceinline__ float e8m0_inv(uint32_t byte) {
  return __builtin_amdgcn_ldexpf(1.0f, 127 - (int)byte);
}
__device__ __forceinline__ float e8m0_val(uint32_t byte) {
  return __builtin_amdgcn_ldexpf(1.0f, (int)byte - 127);
}

// E4M3 code of a non-negative finite fp32 value: nearest, ties to even,
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode_pos(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  uint32_t u = __float_as_uint(v);
  int ex = (int)(u >> 23) - 127;            // v normal in fp32 here unless tiny
  if (ex < -6) {                             // E4M3 subnormal: multiples of 2^-9
    float q = __builtin_rintf(v * 512.0f);   // exact scaling; ties to even
    return (uint32_t)q;                      // 8 is the smallest normal, encoded as 0x08
  }
  // round the fp32 mantissa to 3 bits, nearest even; carry bumps the exponent
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;   // (exp << 3) | m3 in fp32 bias
  uint32_t code = r - ((127u - 7u) << 3);
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return (float)m * (1.0f / 512.0f);
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

}  // namespace sharq
