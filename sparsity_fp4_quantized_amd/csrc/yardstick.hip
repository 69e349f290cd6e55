// Measurement kernels behind bench.py's yardsticks; they are not part of the
// sharq ABI and the hot path never calls them.
//
// What does a kernel that does nothing but FP4 scaled MFMAs reach on this
// GPU?  The published dense FP4 peak assumes the 2.4 GHz peak engine clock;
// under sustained MFMA work on random data the clock settles lower.  Each
// wavefront holds four pairs of random E2M1 operands (drawn from a per-lane
// xorshift state), runs iters x 24 v_mfma_scale_f32_32x32x64_f8f6f4 over six
// accumulators (the tiled dual GEMM's wavefront also updates six 32 x 32
// tiles) with a workgroup barrier every 24, and wavefront 0 of each
// workgroup records how far s_memtime (engine clock) and s_memrealtime
// (100 MHz reference) advanced over the loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_fp4_rate_kernel(float *out, long long *ticks, int iters,
                                                             int random_operands) {
  uint32_t x = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 12345u;
  v8i a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      // E2M1 codes below 8 in every nibble (no sign), so sums cannot cancel
      a[i][j] = random_operands ? (int)(x & 0x77777777u) : 0x22222222;
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      b[i][j] = random_operands ? (int)(x & 0x77777777u) : 0x22222222;
    }
#pragma unroll
    for (int j = 4; j < 8; ++j) a[i][j] = b[i][j] = 0;
  }
  v16f acc[6];
#pragma unroll
  for (int i = 0; i < 6; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  const long long r0 = __builtin_amdgcn_s_memrealtime(), c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 6; ++i)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(i + j) & 3], b[j], acc[i], 4, 4, 0, 100, 0, 100);
    __syncthreads();
  }
  const long long r1 = __builtin_amdgcn_s_memrealtime(), c1 = __builtin_amdgcn_s_memtime();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 6; ++i) s += acc[i][threadIdx.x & 15];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = r1 - r0;
    ticks[2 * blockIdx.x + 1] = c1 - c0;
  }
}

// What does a kernel that only reads reach on this GPU for a given size?
// Each thread reads four 16-byte pieces (a wavefront four contiguous 1 KiB
// runs), all loads issued before any is used; one word per workgroup is
// written so that the loads are kept.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *src, unsigned *out) {
  const size_t base = (size_t)blockIdx.x * 1024 + (threadIdx.x >> 6) * 256 + (threadIdx.x & 63);
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[base + 64 * i];
  unsigned x = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  __shared__ unsigned part[4];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (unsigned)__shfl_xor((int)x, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

// Reads `bytes` bytes of src (a multiple of 16 KiB, 16-byte aligned) once;
// out holds bytes / 16384 words.  Returns the launch's hipError_t.
extern "C" int sharq_yardstick_stream_read(const void *src, size_t bytes, unsigned *out, void *stream) {
  if (src == nullptr || out == nullptr || bytes == 0 || bytes % 16384 != 0 || (uintptr_t)src % 16 != 0)
    return (int)hipErrorInvalidValue;
  stream_read_kernel<<<dim3((unsigned)(bytes / 16384)), dim3(256), 0, (hipStream_t)stream>>>(
      static_cast<const uint4 *>(src), out);
  return (int)hipGetLastError();
}

// workgroups of 256 threads; out holds workgroups * 256 floats, ticks
// 2 * workgroups int64 (per workgroup: 100 MHz ticks, engine clock ticks).
// Returns the launch's hipError_t.
extern "C" int sharq_yardstick_mfma_fp4(int workgroups, int iters, int random_operands, float *out,
                                        long long *ticks, void *stream) {
  if (workgroups <= 0 || iters <= 0 || out == nullptr || ticks == nullptr) return (int)hipErrorInvalidValue;
  mfma_fp4_rate_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream>>>(out, ticks, iters,
                                                                                          random_operands);
  return (int)hipGetLastError();
}
