// Stand-ins for the HIP launch functions, so that the C ABI's host code
// (sharq_abi.cpp: validation, view decoding, dispatch) can be built for the
// host alone with AddressSanitizer and UndefinedBehaviorSanitizer.  Each stub
// counts its calls and checks what the dispatch handed it; nothing touches
// the (fake) device pointers.
#include <hip/hip_runtime.h>

#include "kernels.h"

static int g_launches = 0, g_bad = 0;

extern "C" int sharq_stub_launches(void) { return g_launches; }
extern "C" int sharq_stub_bad(void) { return g_bad; }

namespace sharq {

static hipError_t count(bool ok) {
  ++g_launches;
  if (!ok) ++g_bad;
  return hipSuccess;
}

hipError_t launch_prepare_mx(const PrepArgs &a, hipStream_t) { return count(a.x && a.m > 0 && a.k % 32 == 0); }
hipError_t launch_prepare_silu_mx(const PrepArgs &a, hipStream_t) { return count(a.gate && a.up && a.m > 0); }
hipError_t launch_prepare_nv(const PrepArgs &a, hipStream_t) {
  return count(a.x && a.tensor_scale && a.amax == a.tensor_scale + 1 && a.k % 16 == 0);
}
hipError_t launch_prepare_noalloc(PrepArgs a, int fmt, hipStream_t) { return count(a.x && (fmt == 0 || a.tensor_scale)); }
hipError_t launch_quantize_weight_mx(const QuantArgs &a, hipStream_t) { return count(a.w && a.codes && a.scales); }
hipError_t launch_quantize_weight_nv(const QuantArgs &a, hipStream_t) { return count(a.w && a.tensor_scale); }
hipError_t launch_dual_gemm_mx(const GemmArgs &a, bool, hipStream_t) { return count(a.y && a.k % 128 == 0); }
hipError_t launch_dual_gemm_mx_fp8sp(const GemmArgs &a, hipStream_t) { return count(a.y && a.s_codes && a.meta); }
hipError_t launch_grouped_dual_gemm_mx(const GemmArgs &a, hipStream_t) { return count(a.group_off && a.groups > 0); }
hipError_t launch_dual_gemm_silu_prep_mx(const GemmArgs &a, const PrepArgs &p, hipStream_t) {
  return count(a.n % 2 == 0 && p.s_codes);
}
hipError_t launch_grouped_dual_gemm_silu_prep_mx(const GemmArgs &a, const PrepArgs &p, hipStream_t) {
  return count(a.group_off && p.r_codes);
}
hipError_t launch_dual_gemm_nv(const GemmArgs &a, int, hipStream_t) { return count(a.a_tensor_scale && a.w_tensor_scale); }

}  // namespace sharq
