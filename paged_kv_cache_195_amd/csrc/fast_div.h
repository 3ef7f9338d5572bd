// Division by a run-time divisor fixed for a whole launch (the GQA group
// size) as a multiply-high, an add and a shift, with the multiplier formed
// once on the host.  The method is Granlund and Montgomery's ("Division by
// Invariant Integers using Multiplication", 1994; the round-up form with
// an added dividend): for d >= 1, l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, floor(n / d) = (mulhi(n, m) + n) >> l
// for every 32-bit n, the sum taken in 33 bits.  Dividends here are below
// 2^31, so the sum fits 32 bits.  A loop on the host checks it against
// plain division (tests/host_sanitize/fast_div_check.cpp).
#pragma once

#include <stdint.h>

namespace pa {

struct DivMagic {
  uint32_t m;
  int32_t l;
};

// The multiplier and shift for divisor d (1 <= d < 2^31).
constexpr DivMagic div_magic(uint32_t d) {
  int32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return DivMagic{static_cast<uint32_t>(m), l};
}

// floor(n / d) for 0 <= n < 2^31, given div_magic(d).
constexpr int32_t div_by(int32_t n, DivMagic q) {
  const uint32_t u = static_cast<uint32_t>(n);
  const uint32_t hi = static_cast<uint32_t>((static_cast<uint64_t>(u) * q.m) >> 32);
  return static_cast<int32_t>((hi + u) >> q.l);
}

}  // namespace pa
