// Host build of the preparation's binary64 -> bf16 rounding (the device
// function in prep_block.h), exported for a CPU test that compares it with
// the CPU reference's rounding on every branch (NaN, overflow to Inf, the
// top binade, normal values, the bf16 subnormal range).
#include "prep_block.h"

extern "C" uint32_t host_bf16_of_double(double v) { return sharq::bf16_of_double(v); }
