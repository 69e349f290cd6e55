// Device utilities shared by the MXFP4 and NVFP4-style dual GEMM kernels:
// operand types, the swizzled LDS chunk layout, buffer resources and the
// direct global -> LDS loads (buffer_load ... lds), and the stage wait.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sharq {
namespace gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
// clang vector types (not HIP's uint4 struct) so that staged data stays in registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BK = 128;
constexpr int kThreads = 512;

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

// Expand eight 2:4 groups (8 code bytes, 4 meta bytes) into 32 dense codes.
__device__ __forceinline__ void expand8(uint32_t c_lo, uint32_t c_hi, uint32_t meta, uint32_t out[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = 2 * q + gg;
      const uint32_t cb = ((g < 4 ? c_lo : c_hi) >> (8 * (g & 3))) & 0xFFu;
      const uint32_t s0 = ((meta >> (4 * g)) & 3u) << 2;
      const uint32_t s1 = ((meta >> (4 * g + 2)) & 3u) << 2;
      const uint32_t d16 = ((cb & 15u) << s0) | ((cb >> 4) << s1);
      word |= d16 << (16 * gg);
    }
    out[q] = word;
  }
}

}  // namespace gemm
}  // namespace sharq
