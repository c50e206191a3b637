// Integer division by a divisor fixed for a whole launch, for numerators
// below 2^31, as one 32x32->64-bit multiply and a shift.
//
// For a divisor d >= 1 let l = ceil(log2 d), m = ceil(2^(31+l) / d) and
// sh = 31 + l.  Then 2^(31+l) <= m*d < 2^(31+l) + d <= 2^(31+l) + 2^l, and
// by Theorem 4.2 of Granlund and Montgomery, "Division by invariant integers
// using multiplication" (PLDI 1994), floor(n / d) = floor(n*m / 2^sh) for
// every 0 <= n < 2^31.  Since d > 2^(l-1), m < 2^32, and n*m < 2^63.
//
// Plain C++ (no HIP types), so that the host computes the constants, the
// kernels apply them, and a CPU test checks the same code.
#ifndef FP8BQ_DIV31_HPP
#define FP8BQ_DIV31_HPP

#include <stdint.h>

#if defined(__HIPCC__)
#define FP8BQ_HOST_DEVICE __host__ __device__
#else
#define FP8BQ_HOST_DEVICE
#endif

namespace fp8bq {

struct Div31 {
  uint32_t m;   // ceil(2^sh / d)
  uint32_t sh;  // 31 + ceil(log2 d)
};

// Constants for divisor d (1 <= d < 2^31).
inline Div31 make_div31(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t p = uint64_t(1) << (31 + l);
  Div31 r;
  r.m = static_cast<uint32_t>((p + d - 1) / d);
  r.sh = 31 + l;
  return r;
}

// floor(n / d) for 0 <= n < 2^31.
FP8BQ_HOST_DEVICE inline uint32_t div31(uint32_t n, Div31 d) {
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * d.m) >> d.sh);
}

}  // namespace fp8bq

#endif  // FP8BQ_DIV31_HPP
