// Division of non-negative 31-bit integers by a divisor fixed at launch:
// q = floor(n / d) = (n * m) >> s, with m and s computed once on the host.
// This is the round-up method of Granlund and Montgomery ("Division by
// invariant integers using multiplication", 1994, Theorem 4.2) for N = 31
// bit dividends: with l = ceil(log2 d) and m = ceil(2^(31 + l) / d), m fits
// in 32 bits and the identity holds for every 0 <= n < 2^31.  On the device
// it is a scalar 32x32 -> 64-bit product and a shift, in place of the
// reciprocal-and-correct sequence a run-time divisor otherwise costs.
// Plain integer arithmetic: a host program in the test suite checks it.
// Internal; not installed.
#pragma once

#if defined(__HIPCC__) || defined(__HIP__)
#define MIATTN_FD_HD __host__ __device__
#else
#define MIATTN_FD_HD
#endif

namespace miattn {

struct UDiv {
  unsigned m;  // multiplier, < 2^32
  int s;       // shift, 31 .. 62
};

// d >= 1 (a divisor below 1 is taken as 1)
MIATTN_FD_HD inline UDiv make_udiv(int d) {
  if (d < 1) d = 1;
  int l = 0;
  while ((1LL << l) < d) ++l;  // l = ceil(log2 d)
  const unsigned long long num = 1ULL << (31 + l);
  const unsigned long long m = (num + (unsigned long long)d - 1) / (unsigned long long)d;
  return UDiv{(unsigned)m, 31 + l};
}

// floor(n / d) for 0 <= n < 2^31
MIATTN_FD_HD inline int udiv(int n, UDiv v) {
  return (int)(((unsigned long long)(unsigned)n * v.m) >> v.s);
}

}  // namespace miattn
