// IEEE binary16 conversions for the host side of libsvdq.
//
// Rounding is to nearest, ties to even, in a single step from the source
// type (a binary64 value is not first rounded to binary32). Overflow goes to
// infinity, as IEEE prescribes; callers clamp first where they must not
// overflow.
#pragma once

#include <cmath>
#include <cstdint>
#include <cstring>

namespace svdq {

inline uint16_t f64_to_f16(double x) {
  uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  double a = std::fabs(x);
  if (std::isnan(x)) return 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u;          // >= max + half ulp rounds to inf
  if (a < 0x1p-14) {                                // subnormal range: multiples of 2^-24
    double q = std::nearbyint(std::ldexp(a, 24));   // exact scaling, then RNE
    return sign | static_cast<uint16_t>(q);          // q == 1024 is the smallest normal
  }
  int e;
  std::frexp(a, &e);                                 // a = m 2^e, m in [0.5, 1)
  int E = e - 1;                                     // a = 1.f 2^E, E in [-14, 15]
  double mant = std::nearbyint(std::ldexp(a, 10 - E)) - 1024.0;  // 10 fraction bits, RNE
  if (mant >= 1024.0) {
    mant = 0.0;
    ++E;
  }
  if (E > 15) return sign | 0x7C00u;
  return sign | static_cast<uint16_t>(((E + 15) << 10) | static_cast<int>(mant));
}

inline uint16_t f32_to_f16(float x) { return f64_to_f16(static_cast<double>(x)); }

inline double f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (e == 0) {
    v = std::ldexp(static_cast<double>(m), -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(m + 1024), e - 25);
  }
  return s ? -v : v;
}

inline float f16_to_f32(uint16_t h) { return static_cast<float>(f16_to_f64(h)); }

}  // namespace svdq
