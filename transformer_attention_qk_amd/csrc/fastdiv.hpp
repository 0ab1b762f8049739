// Division by a divisor fixed at launch, as a multiply-high, an add and a shift.
//
// Round-up multiplier method (T. Granlund and P. L. Montgomery, "Division by Invariant Integers
// using Multiplication", PLDI 1994): for a divisor 1 <= d <= 2^31, s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (which fits 32 bits), every 0 <= n < 2^31 satisfies
// n / d == (mulhi(n, m) + n) >> s, where mulhi is the high word of the 64-bit product. Since
// mulhi(n, m) < n, the 32-bit sum cannot wrap for n < 2^31. The kernels use it for the
// head and item indices their workgroups walk through, where a runtime division would cost a
// few dozen scalar instructions per use.
#pragma once

#include <stdint.h>

namespace attn {

struct FastDiv {
  uint32_t d, m, s;

  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
    return (hi + n) >> s;
  }
  __host__ __device__ __forceinline__ uint32_t mod(uint32_t n) const { return n - div(n) * d; }
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

}  // namespace attn
