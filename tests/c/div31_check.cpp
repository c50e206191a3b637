// Checks fp8bq::div31 (the multiply-and-shift division the dequantization
// kernel uses for row, tile-row and tile-column indices) against the C
// division operator.  Exits non-zero and names the first failure.
//
// Exhaustive over every numerator below 2^31 for a few divisors (the
// worst-case error of the method grows with n, and these divisors cover
// small, power-of-two, just-above-a-power-of-two and the largest); edge and
// random numerators for every divisor 1..65536 and random larger ones.
#include <stdio.h>
#include <stdlib.h>

#include "div31.hpp"

static int check(uint32_t n, uint32_t d, fp8bq::Div31 k) {
  if (fp8bq::div31(n, k) != n / d) {
    printf("FAIL n=%u d=%u got=%u want=%u\n", n, d, fp8bq::div31(n, k), n / d);
    return 1;
  }
  return 0;
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd31() {  // splitmix64, top 31 bits
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return static_cast<uint32_t>((z ^ (z >> 31)) >> 33);
}

static int sweep(uint32_t d) {
  const fp8bq::Div31 k = fp8bq::make_div31(d);
  const uint32_t top = 0x7FFFFFFFu;
  const uint32_t edges[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1 < top ? 2 * d - 1 : top,
                            top, top - 1, top - top % d, top - top % d - 1};
  for (uint32_t n : edges) {
    if (n <= top && check(n, d, k)) return 1;
  }
  // the last few multiples below 2^31, where the error term is largest
  for (uint32_t j = 0; j < 64; ++j) {
    const uint64_t base = (uint64_t)(top / d - j) * d;
    if (base > top) continue;
    if (check((uint32_t)base, d, k)) return 1;
    if (base >= 1 && check((uint32_t)(base - 1), d, k)) return 1;
  }
  for (int i = 0; i < 200; ++i) {
    if (check(rnd31(), d, k)) return 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  const bool exhaustive = argc < 2 || argv[1][0] != 'q';
  for (uint32_t d = 1; d <= 65536; ++d) {
    if (sweep(d)) return 1;
  }
  for (int i = 0; i < 200000; ++i) {
    const uint32_t d = rnd31() | 1u;
    if (d > 0 && sweep(d)) return 1;
  }
  for (uint32_t l = 0; l < 31; ++l) {
    const uint32_t p = 1u << l;
    if (sweep(p) || (p > 1 && sweep(p - 1)) || sweep(p + 1)) return 1;
  }
  if (sweep(0x7FFFFFFFu)) return 1;
  if (exhaustive) {
    const uint32_t ds[] = {3u, 375u, 512u, 65537u, 0x7FFFFFFFu};
    for (uint32_t d : ds) {
      // quotient and remainder tracked by counting, with no division
      const fp8bq::Div31 k = fp8bq::make_div31(d);
      uint32_t want = 0, rem = 0;
      for (uint32_t n = 0; n < 0x80000000u; ++n) {
        if (fp8bq::div31(n, k) != want) {
          printf("FAIL exhaustive n=%u d=%u\n", n, d);
          return 1;
        }
        if (++rem == d) {
          rem = 0;
          ++want;
        }
      }
    }
  }
  printf("div31 ok%s\n", exhaustive ? " (exhaustive divisors included)" : "");
  return 0;
}
