// Host-side helpers shared by the packer and the quantizer: IEEE binary16 <->
// binary64 conversion written from the format definition, and a small
// parallel loop over host threads.
#pragma once

#include <math.h>
#include <stdint.h>

#include <thread>
#include <vector>

namespace lutgemm {
namespace host {

// ---- IEEE binary16 <-> binary64, from the format definition ------------------
// binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;
// exponent field 0 = zero/subnormal (value = fraction * 2^-24),
// exponent field 31 = infinity/NaN.

inline bool f16_is_finite(uint16_t h) { return (h & 0x7C00u) != 0x7C00u; }

inline double f16_to_f64(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 0x1F;
  const int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f | 0x400), e - 25);
  }
  return sign ? -v : v;
}

// Round a finite binary64 value to the nearest binary16, ties to even.
// Values at or beyond the overflow threshold become infinity.
inline uint16_t f64_to_f16_rne(double v) {
  const uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -14)) {
    // subnormal range: integer multiple of 2^-24 (rint rounds ties to even)
    double m = rint(ldexp(a, 24));
    return sign | (uint16_t)m;  // m == 1024 is the smallest normal, encoded alike
  }
  int e2;
  frexp(a, &e2);      // a = f * 2^e2, f in [0.5, 1)
  int e = e2 - 1;     // a in [2^e, 2^(e+1))
  double m = rint(ldexp(a, 10 - e));  // in [1024, 2048]
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e + 15 >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)m - 1024);
}

// Run body(lo, hi) over [0, n) split across a few host threads.
template <class F>
void parallel_for(int64_t n, F body) {
  unsigned hw = std::thread::hardware_concurrency();
  int64_t nt = hw ? (int64_t)hw : 1;
  if (nt > 16) nt = 16;
  if (n < 64 || nt <= 1) {
    body(0, n);
    return;
  }
  if (nt > n) nt = n;
  std::vector<std::thread> th;
  th.reserve((size_t)nt);
  for (int64_t t = 0; t < nt; ++t) {
    int64_t lo = n * t / nt, hi = n * (t + 1) / nt;
    th.emplace_back([=] { body(lo, hi); });
  }
  for (auto& t : th) t.join();
}

}  // namespace host
}  // namespace lutgemm
