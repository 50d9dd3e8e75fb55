// fp64 exp for the sampler's weights exp((z - max z) / T), arguments <= 0.
//
// Table-driven method of P. T. P. Tang, "Table-driven implementation of the
// exponential function in IEEE floating-point arithmetic", ACM TOMS 15(2),
// 1989, in base 2 with a 256-entry table: the caller forms
//   y = (z - m) * (256 / (T ln 2))        (one rounding of a double product)
// and exp2_256(y) = 2^(y/256) splits y = 256 k + j + t (k, j integers,
// 0 <= j < 256, |t| <= 1/2, t exact by Sterbenz's lemma):
//   2^(y/256) = 2^k * 2^(j/256) * exp(t ln2 / 256),
// with exp(r) - 1 from its degree-4 Taylor polynomial (|r| <= ln2/512, so the
// truncation stays below 4e-17) and 2^(j/256) from a table the caller fills
// with exp2(j/256).  Relative error of exp2_256 for an exact y stays below
// ~3e-16; the rounding of y adds |y| ln2/256 * 2^-53, about 1.1e-16 per unit
// of |(z - m)/T| -- the same order as forming (z - m)/T in double at all.
// Both are far inside the 1e-12 decision margins of the sampler.
//
// The header compiles for the device (hipcc) and for host-side accuracy tests.
#pragma once
#include <math.h>

#if defined(__HIPCC__)
#define SV_HD __host__ __device__ __forceinline__
#else
#define SV_HD static inline
#endif

namespace sv {

constexpr double kY256PerLn2 = 369.3299304675746;       // 256 / ln 2
// Taylor coefficients of exp(t * ln2/256) - 1 in powers of t: (ln2/256)^i / i!
constexpr double kE1 = 2.7076061740622863e-03;
constexpr double kE2 = 3.6655655969101062e-06;
constexpr double kE3 = 3.3083026805413713e-09;
constexpr double kE4 = 2.2393951908751570e-12;
// Below this y every result rounds to +0 (2^(y/256) < 2^-1075).
constexpr double kYMin = -1076.0 * 256.0;

// 2^(y/256) for y <= 0 (including -inf; NaN gives 0 as well); `tab[j]` =
// 2^(j/256), j = 0..255.  Branch-free: the clamp at kYMin makes every
// argument at or below it (and NaN, which fmax drops) come out as +0.
SV_HD double exp2_256(double y_in, const double* tab) {
    const double y = fmax(y_in, kYMin);
    const double kd = rint(y);
    const double t = y - kd;
    double p = fma(t, kE4, kE3);
    p = fma(t, p, kE2);
    p = fma(t, p, kE1);
    p = p * t;  // exp(t ln2/256) - 1
    const int k = static_cast<int>(kd);
    const double b = tab[k & 255];
    return ldexp(fma(b, p, b), k >> 8);  // arithmetic shift: floor(k / 256)
}

}  // namespace sv
