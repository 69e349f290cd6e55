// NVFP4-style dual GEMM (emulated scales): not built yet.
#include "kernels.h"

namespace sharq {
hipError_t launch_dual_gemm_nv(const GemmArgs &, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace sharq
