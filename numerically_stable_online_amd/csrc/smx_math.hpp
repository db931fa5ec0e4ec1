// smx_math.hpp — scalar arithmetic shared by the row-softmax kernels.
//
// Everything here is plain IEEE fp32 and fp64 arithmetic (add, multiply,
// fused multiply-add, conversion, round-to-integer, scale by a power of
// two), so the same code compiles for gfx950 and, for testing, for the host
// CPU, where it gives the same bits (the hardware base-2 exponential, which
// the exp_dd forms take as an argument, aside).
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define SMX_HD __host__ __device__ inline
#else
#define SMX_HD inline
#endif

namespace smx {

SMX_HD uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
SMX_HD float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Exact difference a - b = hi + lo (Knuth's branch-free two-sum on a, -b).
SMX_HD void two_diff(float a, float b, float& hi, float& lo) {
  const float s = a - b;
  const float bb = s - a;
  lo = (a - (s - bb)) + (-b - bb);
  hi = s;
}

// Exact sum a + b = hi + lo.
SMX_HD void two_sum(float a, float b, float& hi, float& lo) {
  const float s = a + b;
  const float bb = s - a;
  lo = (a - (s - bb)) + (b - bb);
  hi = s;
}

// exp(dh + dl) * 2^64 for dh <= 0, |dl| <= ulp(dh), accurate to about one
// unit in the last place.
//
// The method is the vectorized-exp recipe of "Softmax numerics
// architecture", section "On CPU, and the pitfalls worth naming": exp(z) =
// 2^(z log2 e), an integer part n taken out as a power of two written into
// the exponent, a polynomial on the remainder. The remainder uses Cody and
// Waite's two-constant reduction r = (dh - n*ln2_hi) - n*ln2_lo + dl; with
// ln2_hi = fl(ln 2) and |n| <= 174, the fused first step is exact, so the
// only error left in r is that of the tiny n*ln2_lo term. The polynomial is
// the degree-7 Taylor series of e^r on |r| <= 0.35, whose truncation error
// (< 8e-9 relative) is below half an ulp.
//
// The result is returned scaled by 2^64 so that exp(d) stays a normal fp32
// number down to d = -131: a later multiply by 2^-64 / l then rounds a
// subnormal probability once, instead of twice. d < -120 gives 0 (the
// probability it feeds is below 2^-150 / l and rounds to zero anyway).
SMX_HD float exp_biased64(float dh, float dl) {
  constexpr float kLog2e = 1.44269502162933349609375f;        // fl(log2 e)
  constexpr float kLn2Hi = 0.693147182464599609375f;          // fl(ln 2)
  constexpr float kLn2Lo = -1.9046542999577002e-09f;          // ln 2 - kLn2Hi
  constexpr float c2 = 0.5f;
  constexpr float c3 = 0.16666666666666666f;
  constexpr float c4 = 0.041666666666666664f;
  constexpr float c5 = 0.008333333333333333f;
  constexpr float c6 = 0.001388888888888889f;
  constexpr float c7 = 0.0001984126984126984f;
  if (!(dh >= -120.0f)) return 0.0f;
  const float n = __builtin_rintf(dh * kLog2e);
  float r = __builtin_fmaf(-n, kLn2Hi, dh);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  r = r + dl;
  float p = c7;
  p = __builtin_fmaf(p, r, c6);
  p = __builtin_fmaf(p, r, c5);
  p = __builtin_fmaf(p, r, c4);
  p = __builtin_fmaf(p, r, c3);
  p = __builtin_fmaf(p, r, c2);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n + 64);
}

// exp(a - b) for a <= b, unscaled, with the factor exactly 1 when a == b
// (this covers -inf == -inf: the side holding the larger maximum of a merge
// keeps its sum unchanged, so an empty summary (-inf, 0) is an identity).
SMX_HD float exp_diff(float a, float b) {
  if (a == b) return 1.0f;
  float hi, lo;
  two_diff(a, b, hi, lo);
  if (!(hi >= -120.0f)) return 0.0f;
  return exp_biased64(hi, lo) * 5.42101086242752217e-20f;  // * 2^-64
}

// The same factor in the 2^64 scale: exp(a - b) 2^64 for a <= b, exactly
// 2^64 when a == b and 0 below a - b = -120. A merge that multiplies a sum
// by it keeps the sum's relative precision down to a - b = -120, where the
// unscaled factor is subnormal below -87 and carries only the subnormal
// spacing's absolute precision; the loss of a confident cross-entropy row
// is made of exactly such far-below terms.
SMX_HD float exp_diff_b64(float a, float b) {
  if (a == b) return 18446744073709551616.0f;
  float hi, lo;
  two_diff(a, b, hi, lo);
  return exp_biased64(hi, lo);  // 0 below -120, for -inf and for NaN
}

// exp(x - m) for fp32 x <= m, with the difference taken in fp64, where it is
// exact (two fp32 values need at most 53 bits unless m is tiny and x far
// below it, and then it is rounded to 2^-53 relative, far below what the
// result keeps). An fp32 value t near (x - m) log2 e (any nearby value serves)
// is the point the base-2 exponential is taken at, and the rest of the
// argument, r = (x - m) - t ln 2, is formed in fp64 from the exact product
// and rounded once. |r| < 2^-15, so 2^t (1 + r) misses e^(x - m) by under
// 2^-31 relative: the result carries the base-2 exponential's own error and
// one rounding. The same splitting as the Cody-Waite step above, with fp64
// instead of a two-constant ln 2 and a two-difference; exp2 is the hardware
// base-2 exponential on the GPU (a correctly rounded stand-in on the host).
constexpr double kLn2d = 0.6931471805599453094;      // ln 2 to double precision
constexpr float kLog2eF = 1.44269502162933349609375f;  // fl(log2 e)

// For sums: exp(x - m), unscaled. x - m is clamped at -160 in fp64 (masked
// lanes, -inf, and values that far below the maximum give exactly 0, since
// 2^(-160 log2 e) flushes), where the clamp is exact even when |m| is so
// large that m - 160 would round back to m in fp32. A NaN x gives 0: the
// caller's maximum carries NaN into the row's poison flag.
template <class Exp2>
SMX_HD float exp_dd_sum(float x, double m64, Exp2 exp2) {
  const double d = __builtin_fmax((double)x - m64, -160.0);
  const float t = (float)d * kLog2eF;
  const float r = (float)__builtin_fma((double)t, -kLn2d, d);
  const float e = exp2(t);
  return __builtin_fmaf(e, r, e);
}

// exp(x - m) * 2^64, a normal fp32 number down to x - m = -120 (as
// exp_biased64), and exactly 0 below that, for -inf and for NaN. The base-2
// argument carries the bias: tb is near (x - m) log2 e + 64, rounded once,
// and r = (x - m) + 64 ln 2 - tb ln 2, so 2^tb (1 + r) = e^(x - m) 2^64
// exactly up to r's truncation.
template <class Exp2>
SMX_HD float exp_dd_b64(float x, double m64, Exp2 exp2) {
  const double d = (double)x - m64;
  const float tb = __builtin_fmaf((float)d, kLog2eF, 64.0f);
  const float r = (float)__builtin_fma((double)tb, -kLn2d, d + 64.0 * kLn2d);
  const float e = exp2(tb);
  const float v = __builtin_fmaf(e, r, e);
  return d >= -120.0 ? v : 0.0f;
}

// Nearest-even rounding of a finite, non-negative fp32 value to bfloat16,
// subnormals included (bfloat16 is the upper half of the fp32 word).
SMX_HD uint32_t bf16_rne(float f) {
  const uint32_t u = f2u(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A compensated fp32 accumulator (Kahan) for non-negative terms.
struct KahanSum {
  float s = 0.0f;
  float c = 0.0f;
  SMX_HD void add(float t) {
    const float y = t - c;
    const float u = s + y;
    c = (u - s) - y;
    s = u;
  }
  // the sum as an unevaluated pair hi + lo
  SMX_HD float hi() const { return s; }
  SMX_HD float lo() const { return -c; }
};

}  // namespace smx
