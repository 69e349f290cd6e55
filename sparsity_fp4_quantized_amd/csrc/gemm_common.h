// Device utilities shared by the MXFP4 and NVFP4-style dual GEMM kernels:
// operand types, the swizzled LDS chunk layout, buffer resources and the
// direct global -> LDS loads (buffer_load ... lds), and the stage wait.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.h"

namespace sharq {
namespace gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BK = 128;   // k per pipeline step

__device__ __forceinline__ v8i as_operand(u32x4 v) {
  v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

// 16-byte slot of logical chunk c of tile row r (tile rows are 64 bytes)
__device__ __forceinline__ int lds_slot(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// One operand array streamed global -> LDS: a buffer resource over its bytes
// from row r0 on (reads past the end return 0), the byte stride between rows
// within a step and the byte stride between 128-k steps.  `bps` is the
// array's bytes per row and step; row-major arrays have ld bytes per row,
// k-step-major ones ld rows per step.
struct OpStream {
  i32x4 rsrc;
  uint32_t row_stride, step;
  uint32_t size;   // the descriptor's byte range: offsets at or past it read 0
};

__device__ __forceinline__ OpStream op_stream(const uint8_t *p, int64_t ld, int ksm, int64_t rows,
                                              int64_t r0, int64_t steps, int64_t bps) {
  OpStream s;
  if (ksm) {
    s.size = (uint32_t)(((steps - 1) * ld + rows - r0) * bps);
    s.rsrc = make_rsrc(p + r0 * bps, s.size);
    s.row_stride = (uint32_t)bps;
    s.step = (uint32_t)(ld * bps);
  } else {
    s.size = (uint32_t)((rows - r0) * ld);
    s.rsrc = make_rsrc(p + r0 * ld, s.size);
    s.row_stride = (uint32_t)ld;
    s.step = (uint32_t)bps;
  }
  return s;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// buffer_load ... lds: the asm has no register result, and its completion is
// waited for explicitly (vmcnt) before the barrier that publishes the stage.
__device__ __forceinline__ void b2l16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void b2l4(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// vmcnt(n) with lgkmcnt and expcnt left alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x3F70 | (N & 0xF) | ((N >> 4) << 14));
}

// A bare barrier: the explicit vmcnt wait before it is the only ordering the
// stage needs, and the memory clobber keeps LDS reads from moving across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Workgroup -> output tile.  Workgroups go to the 8 XCDs round robin (XCD =
// id % 8) and each XCD has its own L2, so XCD x takes a contiguous run of
// tile numbers.  Tiles are numbered in bands of GM tile rows, down the rows
// of a band first, so that a run covers a compact block of tile rows and
// columns: the A rows and W columns of one XCD's tiles stay in its L2.  A
// bijection of [0, gm * gn) for any grid.
__device__ __forceinline__ void xcd_tile(uint32_t id, uint32_t gm, uint32_t gn, uint32_t GM,
                                         uint32_t &tm, uint32_t &tn) {
  const uint32_t T = gm * gn, per = T / 8, rem = T % 8;
  const uint32_t x = id % 8, local = id / 8;
  const uint32_t t = x * per + min(x, rem) + local;
  const uint32_t band = t / (GM * gn), within = t - band * GM * gn;
  const uint32_t rows = min(GM, gm - band * GM);
  tm = band * GM + within % rows;
  tn = within / rows;
}

// fp32 -> bf16, round to nearest even, two values at a time (lo in bits 0-15)
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// One output value at element offset `off`: fp32 into y or, when y16 is set,
// its bf16 rounding into y16.
template <bool NT>
__device__ __forceinline__ void put_y(float *y, uint16_t *y16, int64_t off, float v) {
  if (y16) {
    const uint16_t b = (uint16_t)bf16_pair(v, 0.0f);
    if (NT) __builtin_nontemporal_store(b, y16 + off);
    else y16[off] = b;
  } else {
    if (NT) __builtin_nontemporal_store(v, y + off);
    else y[off] = v;
  }
}

// The fp32 epilogue of a TBM x TBN tile (wavefront (wm, wn): 64 rows x TBN / 2
// columns, 2 x TBN / 64 accumulators of 32 x 32; lane l holds column l % 32,
// rows 8 (r / 4) + 4 h + r % 4), each value times `scale`, non-temporal.
// A tile inside Y (the common case) stores through one wavefront-uniform
// base per value row and a 32-bit lane offset, with no bounds checks; edge
// tiles check every row and column.  (Per-value 64-bit addresses and checks
// were about 12 VALU instructions a value, 96 values a lane: as long as the
// main loop, and with every tile in one round they ran after the MFMAs.)
template <int TBM, int TBN>
__device__ __forceinline__ void store_tile(float *y, int64_t ld, int64_t m0, int64_t n0, int64_t m_end,
                                           int64_t n, int wm, int wn, int h, int li,
                                           const v16f (&acc)[2][TBN / 64], float scale) {
  constexpr int TN = TBN / 64;
  const bool inside = m0 + TBM <= m_end && n0 + TBN <= n && ld < ((int64_t)1 << 22);
  if (inside) {
    float *tile = y + m0 * ld + n0;
    const uint32_t lane_off = ((uint32_t)(wm * 64 + 4 * h) * (uint32_t)ld + (uint32_t)(wn * (TBN / 2) + li)) * 4u;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // rows it 32 + 8 (r / 4) + r % 4 of the wavefront's first row: uniform
        char *row = reinterpret_cast<char *>(tile + (int64_t)(it * 32 + 8 * (r >> 2) + (r & 3)) * ld);
#pragma unroll
        for (int jt = 0; jt < TN; ++jt)
          __builtin_nontemporal_store(acc[it][jt][r] * scale,
                                      reinterpret_cast<float *>(row + lane_off + 128u * jt));
      }
    return;
  }
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < TN; ++jt) {
      const int64_t col = n0 + wn * (TBN / 2) + jt * 32 + li;
      if (col >= n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < m_end) __builtin_nontemporal_store(acc[it][jt][r] * scale, &y[row * ld + col]);
      }
    }
}

// The bf16 form of store_tile above: each value rounded to bf16 (nearest
// even) from the fp32 value store_tile would write.  Values of rows r and
// r + 1 (r even) convert in one instruction; each row of a wavefront's store
// is 32 lanes x 2 bytes, one aligned 64-byte piece when Y's rows are.
template <int TBM, int TBN>
__device__ __forceinline__ void store_tile_bf16(uint16_t *y, int64_t ld, int64_t m0, int64_t n0,
                                                int64_t m_end, int64_t n, int wm, int wn, int h, int li,
                                                const v16f (&acc)[2][TBN / 64], float scale) {
  constexpr int TN = TBN / 64;
  const bool inside = m0 + TBM <= m_end && n0 + TBN <= n && ld < ((int64_t)1 << 22);
  if (inside) {
    uint16_t *tile = y + m0 * ld + n0;
    const uint32_t lane_off = ((uint32_t)(wm * 64 + 4 * h) * (uint32_t)ld + (uint32_t)(wn * (TBN / 2) + li)) * 2u;
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        // rows it 32 + 8 (r / 4) + r % 4 and the one after it: uniform
        char *row0 = reinterpret_cast<char *>(tile + (int64_t)(it * 32 + 8 * (r >> 2) + (r & 3)) * ld);
        char *row1 = row0 + 2 * ld;
#pragma unroll
        for (int jt = 0; jt < TN; ++jt) {
          const uint32_t w = bf16_pair(acc[it][jt][r] * scale, acc[it][jt][r + 1] * scale);
          __builtin_nontemporal_store((uint16_t)w, reinterpret_cast<uint16_t *>(row0 + lane_off + 64u * jt));
          __builtin_nontemporal_store((uint16_t)(w >> 16), reinterpret_cast<uint16_t *>(row1 + lane_off + 64u * jt));
        }
      }
    return;
  }
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < TN; ++jt) {
      const int64_t col = n0 + wn * (TBN / 2) + jt * 32 + li;
      if (col >= n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + it * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < m_end)
          __builtin_nontemporal_store((uint16_t)bf16_pair(acc[it][jt][r] * scale, 0.0f), &y[row * ld + col]);
      }
    }
}

// Host side: tile rows per band for a gm x gn grid of TBM x TBN tiles, so
// that the tiles an XCD runs at one time read about as many A bytes (TBM k
// per tile row, both paths) as W bytes (TBN k / 2 per tile column).  At one
// time an XCD runs its 32 CUs x `resident` workgroups, or its whole share of
// the grid if that is smaller; with several waves of tiles a band as tall as
// the whole share made each wave's block of tiles tall and narrow (the
// NVFP4-style GEMM fetched twice the bytes from beyond the L2).
inline uint32_t xcd_band_rows(int64_t gm, int64_t gn, int tbm, int tbn, int resident) {
  const double per = (double)(gm * gn) / 8.0;
  const double at_once = per < 32.0 * resident ? per : 32.0 * resident;
  const double want = at_once * tbn / (2.0 * tbm);
  uint32_t GM = 1;
  while (GM < gm && (double)(2 * GM) * (2 * GM) <= want * 2.0) GM *= 2;
  return GM;
}

// Expand eight 2:4 groups (8 code bytes, 4 meta bytes) into 32 dense codes.
// Output word q holds groups 2q and 2q + 1, one per 16-bit half, so both are
// placed at once with packed 16-bit shifts: the two code bytes go to bytes 0
// and 2 (v_perm), their low nibbles (code at i0) and high nibbles (code at
// i1) are shifted left by 4 i0 and 4 i1 of their own group.  The meta byte q
// (i0 | i1 << 2 of group 2q, the same of group 2q + 1 in the high nibble) is
// copied to bytes 0 and 2 and shifted right by 0 and 4 per half, which lines
// up 4 i1 in bits 2-3 and i0 in bits 0-1 of each half.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_shl16(uint32_t v, uint32_t s) {
  const u16x2 r = __builtin_bit_cast(u16x2, v) << __builtin_bit_cast(u16x2, s);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ void expand8(uint32_t c_lo, uint32_t c_hi, uint32_t meta, uint32_t out[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t k = 2u * (q & 1);
    const uint32_t x = __builtin_amdgcn_perm(0u, q < 2 ? c_lo : c_hi, k | 0x0C00u | ((k + 1u) << 16) | 0x0C000000u);
    const uint32_t lo = x & 0x000F000Fu, hi = (x >> 4) & 0x000F000Fu;
    const uint32_t y = __builtin_amdgcn_perm(0u, meta, (uint32_t)q | 0x0C00u | ((uint32_t)q << 16) | 0x0C000000u);
    const u16x2 zv = __builtin_bit_cast(u16x2, y) >> u16x2{0, 4};
    const uint32_t z = __builtin_bit_cast(uint32_t, zv);
    out[q] = pk_shl16(lo, (z & 0x00030003u) << 2) | pk_shl16(hi, z & 0x000C000Cu);
  }
}

}  // namespace gemm
}  // namespace sharq
