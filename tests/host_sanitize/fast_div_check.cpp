// Checks csrc/fast_div.h against plain division: every divisor 1..4096 and
// a set of larger ones, each with the dividends around its multiples, near
// 2^31 and spread over [0, 2^31).  Prints "fast_div checks passed" and exits
// 0 when all agree.  Test infrastructure only.
#include <stdio.h>
#include <stdint.h>

#include "fast_div.h"

int main() {
  long long checked = 0, bad = 0;
  auto check = [&](uint32_t d, int32_t n) {
    if (n < 0) return;
    const pa::DivMagic q = pa::div_magic(d);
    const int32_t got = pa::div_by(n, q), want = n / static_cast<int32_t>(d);
    ++checked;
    if (got != want && bad++ < 10) printf("d=%u n=%d: %d != %d\n", d, n, got, want);
  };
  uint64_t x = 88172645463325252ull;  // xorshift64
  auto next = [&]() { x ^= x << 13; x ^= x >> 7; x ^= x << 17; return x; };
  for (uint32_t d = 1; d <= 4096 + 64; ++d) {
    const uint32_t dd = d <= 4096 ? d : static_cast<uint32_t>(next() % 0x7fffffffull) + 1;
    for (int32_t n = 0; n < 2048; ++n) check(dd, n);
    for (int k = 1; k < 64; ++k) {
      const int64_t base = static_cast<int64_t>(dd) * static_cast<int64_t>(next() % (0x7fffffffull / dd + 1));
      for (int64_t o = -2; o <= 2; ++o) {
        const int64_t n = base + o;
        if (n >= 0 && n < 0x7fffffffll) check(dd, static_cast<int32_t>(n));
      }
    }
    for (int32_t o = 0; o < 64; ++o) check(dd, 0x7fffffff - o);
    for (int k = 0; k < 256; ++k) check(dd, static_cast<int32_t>(next() % 0x80000000ull));
  }
  printf("%lld divisions checked, %lld wrong\n", checked, bad);
  if (bad == 0) printf("fast_div checks passed\n");
  return bad == 0 ? 0 : 1;
}
