// MXFP4 dual GEMM with the 2:4 backbone on gfx950's structured-sparse FP8
// MFMA (v_smfmac_f32_32x32x64_fp8_fp8).
//
// "SharQ: Bridging Activation Sparsity and FP4 Quantization for LLM
// Inference" (arXiv:2606.26587), abstract, sentence 4: a sparse FP4 GEMM
// processes the backbone and a dense FP4 GEMM the residual.  gfx950 has a
// block-scaled FP4 MFMA but no structured-sparse MFMA for FP4 operands; its
// sparse MFMAs take fp16, bf16, FP8 or int8.  E2M1 values times a power of two
// are exact in E4M3 over a range of exponents, so the backbone can run on the
// FP8 sparse MFMA once each row of A and of W is rebased to one power of two:
//
//   A row m, block b:  q * 2^(e_mb) = (q * 2^(e_mb - ref_m)) * 2^ref_m
//
// q * 2^d is an exact E4M3 value for every E2M1 q when d lies in [-7, 5]
// (0.5 * 2^-7 = 2^-8 is a multiple of the smallest subnormal 2^-9 and so are
// 1.5 * 2^-7 and 3 * 2^-7; 6 * 2^5 = 192 lies below the largest value under
// either E4M3 bias).  With ref_m = (largest block exponent of the row) - 5,
// every block of a row fits when the row's block exponents span at most 12;
// likewise for each row of W (its sparse-path scale view).  A tile whose A
// and W rows all fit accumulates the backbone on the sparse FP8 MFMA into its
// own accumulator and adds it times 2^(ref_m + ref_n) to the residual's in the
// epilogue (an exact power-of-two scaling unless the result leaves the fp32
// normal range).  Any other tile runs its backbone as the dense kernel does:
// the 2:4 codes expanded to dense FP4 in LDS, on the scaled FP4 MFMA.
//
// Operand layout of the sparse MFMA (probed on one wavefront): lane l holds
// row (A) or column (B) l % 32; A lane half a holds eight 2:4 groups g (two
// FP8 values each, then one index nibble each at bits 4g of the index word);
// group g meets B lane half g / 4, B bytes 16a + 4 (g % 4) .. + 3, and B lane
// half h holds k 32h .. 32h + 31 of the MFMA's 64.  So in the row's numbering
// of the 16 groups of a 64-k window, lane half a takes groups 4a .. 4a + 3
// and 8 + 4a .. 8 + 4a + 3.
//
// Data movement: two LDS stages of raw operands (compressed backbone codes,
// 2:4 indices, residual codes, W codes and the four scale arrays) streamed
// global -> LDS with buffer_load ... lds one 128-k step ahead, and one area of
// converted operands.  Each step: a barrier, the workgroup converts the step's
// backbone and W to FP8 (or expands the backbone, in a fallback tile) into the
// converted area, a barrier, and the MFMAs read both.
#include <stddef.h>

#include "fp4_device.h"
#include "gemm_common.h"
#include "kernels.h"

namespace sharq {
namespace {

using namespace gemm;

constexpr int TB = 128;   // tile rows = tile columns
constexpr int NW = 4;     // wavefronts: 2 x 2, 64 x 64 outputs each

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

struct RawStage {
  uint8_t sc[TB * 32];     // compressed backbone codes, 32 bytes a row
  uint8_t meta[TB * 16];   // 2:4 indices, 16 bytes a row
  u32x4 ar[TB * 4];        // residual codes, 64 bytes a row, chunk-swizzled
  u32x4 w[TB * 4];         // W codes, 64 bytes a row, chunk-swizzled
  uint32_t sas[TB], sar[TB], sws[TB], swd[TB];
};

struct ConvArea {
  u32x4 a8[TB * 4];        // FP8 backbone: chunk 2s + a = window s, lane half a (or dense FP4 codes)
  uint32_t idx[TB * 4];    // index word of window s, lane half a: [row][2s + a]
  u32x4 w8[TB * 8];        // FP8 W: 128 bytes a column in k order, chunk c at c ^ (col & 7)
};

__device__ __forceinline__ int w8_slot(int col, int c) { return col * 8 + (c ^ (col & 7)); }

// 2^d as the fp32 scale operand of the conversion (d in [-126, 127])
__device__ __forceinline__ float pow2f(int d) { return __uint_as_float((uint32_t)(d + 127) << 23); }

// Four E2M1 codes (two bytes of `word`, selected by SEL) times 2^d as four
// FP8 bytes, in code order: exact, since every q 2^d is an E4M3 value.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x4_to_fp8(uint32_t word, float scale) {
  const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 2 * SEL);
  const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, scale, 2 * SEL + 1);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(lo.x, lo.y, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(hi.x, hi.y, r, true);
  return (uint32_t)r;
}

struct Loads {
  // 16-byte loads: compressed codes (4: 32 rows each), meta (2: 64 rows),
  // residual (8: 16 rows), W (8: 16 rows); 4-byte loads: the four scale
  // arrays (2 each: 64 rows)
  static constexpr int kChunks = 22, kScales = 8;
  static constexpr int kChunkPer = (kChunks + NW - 1) / NW, kScalePer = kScales / NW;
  i32x4 rsrc[kChunkPer + kScalePer];
  uint32_t step[kChunkPer + kScalePer], voff[kChunkPer + kScalePer], lds[kChunkPer + kScalePer];
  bool real[kChunkPer];
};

__device__ __forceinline__ void plan(const GemmArgs &a, int64_t m0, int64_t n0, int wave, int lane, Loads &L) {
  const int64_t steps = a.k / BK;
  const OpStream sc = op_stream(a.s_codes, a.ld_sc, a.s_ksm, a.m, m0, steps, 32);
  const OpStream sm = op_stream(a.meta, a.ld_meta, a.s_ksm, a.m, m0, steps, 16);
  const OpStream ar = op_stream(a.r_codes, a.ld_rc, a.r_ksm, a.m, m0, steps, 64);
  const OpStream w = op_stream(a.w_codes, a.ld_wc, a.w_ksm, a.n, n0, steps, 64);
  const OpStream sas = op_stream(a.s_scales, a.ld_ss, a.s_ksm, a.m, m0, steps, 4);
  const OpStream sar = op_stream(a.r_scales, a.ld_rs, a.r_ksm, a.m, m0, steps, 4);
  const OpStream sws = op_stream(a.ws_scales, a.ld_wss, a.w_ksm, a.n, n0, steps, 4);
  const OpStream swd = op_stream(a.wd_scales, a.ld_wds, a.w_ksm, a.n, n0, steps, 4);
  const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lane >> 4) & 3);
#pragma unroll
  for (int j = 0; j < Loads::kChunkPer; ++j) {
    const int q = wave + NW * j;
    L.real[j] = q < Loads::kChunks;
    OpStream o = sc;
    uint32_t voff = 0, lds = 0;
    if (q < 4) {
      voff = (uint32_t)(32 * q + (lane >> 1)) * sc.row_stride + (lane & 1) * 16;
      lds = (uint32_t)offsetof(RawStage, sc) + 1024u * q;
    } else if (q < 6) {
      o = sm;
      voff = (uint32_t)(64 * (q - 4) + lane) * sm.row_stride;
      lds = (uint32_t)offsetof(RawStage, meta) + 1024u * (q - 4);
    } else if (q < 14) {
      o = ar;
      voff = (uint32_t)(16 * (q - 6) + lrow) * ar.row_stride + lchunk * 16;
      lds = (uint32_t)offsetof(RawStage, ar) + 1024u * (q - 6);
    } else {
      o = w;
      voff = (uint32_t)(16 * (q - 14) + lrow) * w.row_stride + lchunk * 16;
      lds = (uint32_t)offsetof(RawStage, w) + 1024u * (q - 14);
    }
    L.rsrc[j] = o.rsrc;
    L.step[j] = o.step;
    L.voff[j] = voff;
    L.lds[j] = lds;
  }
#pragma unroll
  for (int j = 0; j < Loads::kScalePer; ++j) {
    const int q = wave + NW * j;           // 0 .. 7
    const int arr = q >> 1, half = q & 1;
    const OpStream o = arr == 0 ? sas : arr == 1 ? sar : arr == 2 ? sws : swd;
    const uint32_t base = arr == 0 ? (uint32_t)offsetof(RawStage, sas) : arr == 1 ? (uint32_t)offsetof(RawStage, sar)
                        : arr == 2 ? (uint32_t)offsetof(RawStage, sws) : (uint32_t)offsetof(RawStage, swd);
    const int k = Loads::kChunkPer + j;
    L.rsrc[k] = o.rsrc;
    L.step[k] = o.step;
    L.voff[k] = (uint32_t)(64 * half + lane) * o.row_stride;
    L.lds[k] = base + 256u * half;
  }
}

__device__ __forceinline__ void issue(const Loads &L, int kt, const RawStage &S) {
  const uint32_t base = lds_addr(&S), t = (uint32_t)kt;
#pragma unroll
  for (int j = 0; j < Loads::kChunkPer; ++j)
    if (L.real[j]) b2l16(L.rsrc[j], L.voff[j], t * L.step[j], base + L.lds[j]);
#pragma unroll
  for (int j = 0; j < Loads::kScalePer; ++j) {
    const int k = Loads::kChunkPer + j;
    b2l4(L.rsrc[k], L.voff[k], t * L.step[k], base + L.lds[k]);
  }
}

// Rebasing reference of one operand row over the whole K: the largest block
// exponent byte minus 5; `fits` when every block byte lies within 12 of the
// largest.  Rows past the operand's end fit.
__device__ __forceinline__ void row_reference(const uint8_t *scales, int64_t ld, int ksm, int64_t row, int64_t rows,
                                              int64_t k, int &ref, bool &fits) {
  ref = 0;
  fits = true;
  if (row >= rows) return;
  uint32_t mx = 0, mn = 255;
  const int64_t steps = k / BK;
  for (int64_t t = 0; t < steps; ++t) {
    const uint32_t v = *reinterpret_cast<const uint32_t *>(scales + arr_off(row, t, ld, ksm, 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t b = (v >> (8 * i)) & 0xFFu;
      mx = max(mx, b);
      mn = min(mn, b);
    }
  }
  ref = (int)mx - 5;
  fits = mx - mn <= 12;
}

template <bool FP8>
__device__ __forceinline__ void convert(const RawStage &R, ConvArea &C, const int *ref_a, const int *ref_w, int tid) {
  // backbone: row tid / 2, 64-k window s = tid % 2 (16 groups, blocks 2s and 2s + 1)
  {
    const int row = tid >> 1, s = tid & 1;
    const u32x4 codes = *reinterpret_cast<const u32x4 *>(R.sc + row * 32 + 16 * s);
    const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
    const u32x2 mw = *reinterpret_cast<const u32x2 *>(R.meta + row * 16 + 8 * s);
    if constexpr (FP8) {
      const uint32_t sb = R.sas[row];
      const int ref = ref_a[row];
      const float s0 = pow2f((int)((sb >> (16 * s)) & 0xFFu) - ref);
      const float s1 = pow2f((int)((sb >> (16 * s + 8)) & 0xFFu) - ref);
      // code word i holds groups 4i .. 4i + 3 (two codes each): 8 FP8 bytes
      uint32_t f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = i < 2 ? s0 : s1;
        f[2 * i] = fp4x4_to_fp8<0>(cw[i], sc);
        f[2 * i + 1] = fp4x4_to_fp8<1>(cw[i], sc);
      }
      // lane half 0: groups 0-3 and 8-11; lane half 1: groups 4-7 and 12-15
      C.a8[lds_slot(row, 2 * s)] = u32x4{f[0], f[1], f[4], f[5]};
      C.a8[lds_slot(row, 2 * s + 1)] = u32x4{f[2], f[3], f[6], f[7]};
      // index words: the nibbles of the same groups (meta halfwords 0 / 2 and 1 / 3)
      C.idx[row * 4 + 2 * s] = (mw.x & 0xFFFFu) | (mw.y << 16);
      C.idx[row * 4 + 2 * s + 1] = (mw.x >> 16) | (mw.y & 0xFFFF0000u);
    } else {
      // dense FP4: blocks 2s and 2s + 1 (chunks of the dense layout)
      uint32_t d0[4], d1[4];
      expand8(cw[0], cw[1], mw.x, d0);
      expand8(cw[2], cw[3], mw.y, d1);
      C.a8[lds_slot(row, 2 * s)] = u32x4{d0[0], d0[1], d0[2], d0[3]};
      C.a8[lds_slot(row, 2 * s + 1)] = u32x4{d1[0], d1[1], d1[2], d1[3]};
    }
  }
  if constexpr (FP8) {
    // W: column tid / 2, window s = tid % 2 (blocks 2s, 2s + 1: 64 codes)
    const int col = tid >> 1, s = tid & 1;
    const uint32_t sb = R.sws[col];
    const int ref = ref_w[col];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int blk = 2 * s + b;
      const u32x4 cw = R.w[lds_slot(col, blk)];
      const float sc = pow2f((int)((sb >> (8 * blk)) & 0xFFu) - ref);
      const uint32_t x[4] = {cw.x, cw.y, cw.z, cw.w};
      uint32_t f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = fp4x4_to_fp8<0>(x[i], sc);
        f[2 * i + 1] = fp4x4_to_fp8<1>(x[i], sc);
      }
      // 32 k of the block = 32 FP8 bytes = chunks 2 blk and 2 blk + 1
      C.w8[w8_slot(col, 2 * blk)] = u32x4{f[0], f[1], f[2], f[3]};
      C.w8[w8_slot(col, 2 * blk + 1)] = u32x4{f[4], f[5], f[6], f[7]};
    }
  }
}

// One 128-k step of wavefront (wm, wn): 64 x 64 outputs, tiles it, jt of 32 x 32.
template <bool FP8>
__device__ __forceinline__ void mfma_step(const RawStage &R, const ConvArea &C, v16f (&acc_r)[2][2],
                                          v16f (&acc_s)[2][2], int wm, int wn, int h, int li) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    // residual (and, in a fallback tile, the expanded backbone): FP4 x FP4,
    // lane half h takes block 2h + s
    const int c = 2 * h + s;
    v8i ar[2], bw[2];
    int sar[2], swd[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int r = wm * 64 + it * 32 + li;
      ar[it] = as_operand(R.ar[lds_slot(r, c)]);
      sar[it] = (int)(R.sar[r] >> (16 * h));
    }
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const int r = wn * 64 + jt * 32 + li;
      bw[jt] = as_operand(R.w[lds_slot(r, c)]);
      swd[jt] = (int)(R.swd[r] >> (16 * h));
    }
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        if (s == 0)
          acc_r[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ar[it], bw[jt], acc_r[it][jt], 4, 4, 0, sar[it], 0, swd[jt]);
        else
          acc_r[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ar[it], bw[jt], acc_r[it][jt], 4, 4, 1, sar[it], 1, swd[jt]);
      }
    if constexpr (FP8) {
      // backbone: 64-k window s on the sparse FP8 MFMA
      v4i a8[2];
      int idx[2];
      v8i b8[2];
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int r = wm * 64 + it * 32 + li;
        const u32x4 v = C.a8[lds_slot(r, 2 * s + h)];
        a8[it] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        idx[it] = (int)C.idx[r * 4 + 2 * s + h];
      }
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const int col = wn * 64 + jt * 32 + li;
        const u32x4 lo = C.w8[w8_slot(col, 4 * s + 2 * h)];
        const u32x4 hi = C.w8[w8_slot(col, 4 * s + 2 * h + 1)];
        b8[jt] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
          acc_s[it][jt] = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a8[it], b8[jt], acc_s[it][jt], idx[it], 0, 0);
    } else {
      // backbone expanded to dense FP4 in the converted area, scaled FP4 MFMA
      v8i as[2], bw2[2];
      int sas[2], sws[2];
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int r = wm * 64 + it * 32 + li;
        as[it] = as_operand(C.a8[lds_slot(r, c)]);
        sas[it] = (int)(R.sas[r] >> (16 * h));
      }
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const int r = wn * 64 + jt * 32 + li;
        bw2[jt] = as_operand(R.w[lds_slot(r, c)]);
        sws[jt] = (int)(R.sws[r] >> (16 * h));
      }
#pragma unroll
      for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          if (s == 0)
            acc_r[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as[it], bw2[jt], acc_r[it][jt], 4, 4, 0, sas[it], 0, sws[jt]);
          else
            acc_r[it][jt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(as[it], bw2[jt], acc_r[it][jt], 4, 4, 1, sas[it], 1, sws[jt]);
        }
    }
  }
}

template <bool FP8>
__device__ __forceinline__ void main_loop(const Loads &L, RawStage (&raw)[2], ConvArea &conv, const int *ref_a,
                                          const int *ref_w, v16f (&acc_r)[2][2], v16f (&acc_s)[2][2], int ksteps,
                                          int wm, int wn, int h, int li) {
  const int tid = threadIdx.x;
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = kt & 1;
    // step kt's raw operands have landed; every wavefront is done with the
    // converted area and with the other raw stage (step kt - 1)
    wait_vmcnt<0>();
    stage_barrier();
    if (kt + 1 < ksteps) issue(L, kt + 1, raw[cur ^ 1]);
    convert<FP8>(raw[cur], conv, ref_a, ref_w, tid);
    __syncthreads();
    mfma_step<FP8>(raw[cur], conv, acc_r, acc_s, wm, wn, h, li);
  }
}

__global__ __launch_bounds__(64 * NW, 2) void dual_gemm_fp8sp_kernel(GemmArgs a, uint32_t band) {
  __shared__ RawStage raw[2];
  __shared__ ConvArea conv;
  __shared__ int ref_a[TB], ref_w[TB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, li = lane & 31;
  uint32_t tm, tn;
  xcd_tile(blockIdx.x, (uint32_t)((a.m + TB - 1) / TB), (uint32_t)((a.n + TB - 1) / TB), band, tm, tn);
  const int64_t m0 = (int64_t)tm * TB, n0 = (int64_t)tn * TB;
  const int ksteps = (int)(a.k / BK);

  Loads L;
  plan(a, m0, n0, wave, lane, L);
  issue(L, 0, raw[0]);

  // the tile's rebasing references, while step 0 streams in
  int ref;
  bool fits;
  if (tid < TB) row_reference(a.s_scales, a.ld_ss, a.s_ksm, m0 + tid, a.m, a.k, ref, fits);
  else row_reference(a.ws_scales, a.ld_wss, a.w_ksm, n0 + tid - TB, a.n, a.k, ref, fits);
  if (tid < TB) ref_a[tid] = ref;
  else ref_w[tid - TB] = ref;
  const bool fp8 = __syncthreads_and(fits) != 0;

  v16f acc_r[2][2], acc_s[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc_r[i][j][r] = 0.0f;
        acc_s[i][j][r] = 0.0f;
      }
  if (fp8) main_loop<true>(L, raw, conv, ref_a, ref_w, acc_r, acc_s, ksteps, wm, wn, h, li);
  else main_loop<false>(L, raw, conv, ref_a, ref_w, acc_r, acc_s, ksteps, wm, wn, h, li);

  // Y = residual + backbone * 2^(ref_m + ref_n - 2 * 127): both scale bytes
  // carry the E8M0 bias
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      const int cl = wn * 64 + jt * 32 + li;
      const int64_t col = n0 + cl;
      if (col >= a.n) continue;
      const int ew = ref_w[cl] - 254;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = wm * 64 + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t row = m0 + rl;
        if (row >= a.m) continue;
        float v = acc_r[it][jt][r];
        if (fp8) v += __builtin_ldexpf(acc_s[it][jt][r], ref_a[rl] + ew);
        put_y<true>(a.y, a.y16, row * a.ld_y + col, v);
      }
    }
}

}  // namespace

hipError_t launch_dual_gemm_mx_fp8sp(const GemmArgs &a, hipStream_t s) {
  const int64_t gm = (a.m + TB - 1) / TB, gn = (a.n + TB - 1) / TB;
  dual_gemm_fp8sp_kernel<<<dim3((unsigned)(gm * gn)), dim3(64 * NW), 0, s>>>(a, xcd_band_rows(gm, gn, TB, TB, 2));
  return hipGetLastError();
}

}  // namespace sharq
