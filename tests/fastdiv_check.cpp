// Host check of fastdiv.h: udiv(n, make_udiv(d)) == n / d for every divisor
// 1 .. 5000 against dividends around each multiple of d up to 2^31 - 1 and
// a sweep, and for divisors up to 2^31 - 1 at sampled points.  Prints one
// line per failure and exits with status 1 if any.
#include <cstdint>
#include <cstdio>

#include "fastdiv.h"

using namespace miattn;

static int g_fails = 0;
static void check(int n, int d) {
  const int q = udiv(n, make_udiv(d));
  if (q != n / d && g_fails++ < 20)
    std::printf("FAIL n=%d d=%d got %d want %d\n", n, d, q, n / d);
}

int main() {
  const int top = 2147483647;
  for (int d = 1; d <= 5000; ++d) {
    for (int n = 0; n < 4 * d + 10; ++n) check(n, d);
    for (long long k = d; k <= top; k = k * 3 + 7) {
      for (int e = -2; e <= 2; ++e) {
        const long long n = (k / d) * d + e;
        if (n >= 0 && n <= top) check((int)n, d);
      }
    }
    for (int e = 0; e < 4; ++e) check(top - e, d);
  }
  unsigned long long x = 88172645463325252ULL;  // xorshift64
  for (int i = 0; i < 2000000; ++i) {
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    const int d = (int)((x >> 33) % 2147483647ULL) + 1;
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    const int n = (int)(x >> 33);
    check(n, d);
    check(n, (d & 0xFFFF) + 1);
  }
  if (g_fails) {
    std::printf("%d failures\n", g_fails);
    return 1;
  }
  std::printf("fastdiv: all checks passed\n");
  return 0;
}
