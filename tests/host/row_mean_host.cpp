// Host build of the preparation's row mean (prep_block.h) for
// tests/test_host_rounding.py: counts the (ss, k) cases where it differs from
// the IEEE binary32 quotient ss / k.
#include <cstdint>
#include <cstring>

#include "prep_block.h"

namespace {
float from_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
uint32_t bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
uint64_t next(uint64_t &s) {   // xorshift64*
  s ^= s >> 12;
  s ^= s << 25;
  s ^= s >> 27;
  return s * 0x2545F4914F6CDD1Dull;
}
}  // namespace

// k = 32, 64, .., kmax; per k `samples` random ss over every binade from
// 2^-110 to 2^110 (both sides of each range limit) plus structured cases:
// exact quotients, all-ones significands, the range limits and their
// neighbours, zero, Inf and NaN.  Returns the number of mismatches (NaN
// matches NaN); *cases receives the number of cases.
extern "C" int64_t host_row_mean_mismatches(int64_t kmax, int64_t samples, uint64_t seed,
                                            int64_t *cases) {
  int64_t bad = 0, n = 0;
  uint64_t s = seed | 1;
  auto check = [&](float ss, float kf, float inv_k) {
    const float got = sharq::row_mean_of(ss, kf, inv_k), want = ss / kf;
    ++n;
    if (!(bits(got) == bits(want) || (got != got && want != want))) ++bad;
  };
  for (int64_t k = 32; k <= kmax; k += 32) {
    const float kf = (float)k, inv_k = 1.0f / kf;
    for (int64_t i = 0; i < samples; ++i) {
      const uint64_t r = next(s);
      const uint32_t e = 127 - 110 + (uint32_t)(r % 221);   // binades 2^-110 .. 2^110
      check(from_bits((e << 23) | (uint32_t)((r >> 20) & 0x7FFFFF)), kf, inv_k);
    }
    for (uint32_t j = 1; j <= 64; ++j) {
      check((float)j * kf, kf, inv_k);                                  // exact quotients
      check(from_bits(bits((float)j * kf) + 1), kf, inv_k);
      check(from_bits(bits((float)j * kf) - 1), kf, inv_k);
    }
    for (uint32_t e = 127 - 100; e <= 127 + 100; e += 7) check(from_bits((e << 23) | 0x7FFFFF), kf, inv_k);
    for (float lim : {0x1p-100f, 0x1p100f}) {
      check(lim, kf, inv_k);
      check(from_bits(bits(lim) - 1), kf, inv_k);
      check(from_bits(bits(lim) + 1), kf, inv_k);
    }
    check(0.0f, kf, inv_k);
    check(from_bits(0x7F800000u), kf, inv_k);
    check(from_bits(0x7FC00000u), kf, inv_k);
    check(from_bits(1u), kf, inv_k);
  }
  *cases = n;
  return bad;
}
