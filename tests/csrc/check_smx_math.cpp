// Host build of the kernels' scalar arithmetic (smx_math.hpp), checked
// against libm's double-precision exp. Prints one line of results.
//   check_smx_math <stride>
// walks every stride-th fp32 value d in [-120, 0] with dl = 0, plus a seeded
// set of (dh, dl) pairs formed as exact differences of two fp32 values; then
// the fp64-difference forms (exp_dd_b64, exp_dd_sum) on the same walk and on
// seeded pairs (x, m) of every magnitude, with a correctly rounded base-2
// exponential standing in for the hardware one, and their special cases.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "smx_math.hpp"

static double ulp_err(float got, double ref) {
  // error in units of the fp32 spacing at the reference (subnormal spacing
  // below 2^-126 in the biased domain never occurs here)
  int e;
  std::frexp(ref, &e);
  double ulp = std::ldexp(1.0, e - 24);
  return std::fabs((double)got - ref) / ulp;
}

int main(int argc, char** argv) {
  const unsigned stride = argc > 1 ? (unsigned)std::atoi(argv[1]) : 1;
  double worst = 0.0, worst_d = 0.0;
  long n = 0;
  // all negative floats down to -120, by bit pattern
  const uint32_t lo_bits = 0x80000000u, hi_bits = smx::f2u(-120.0f);
  for (uint64_t b = lo_bits; b <= hi_bits; b += stride) {
    float d = smx::u2f((uint32_t)b);
    double ref = std::ldexp(std::exp((double)d), 64);
    float got = smx::exp_biased64(d, 0.0f);
    double u = ulp_err(got, ref);
    if (u > worst) { worst = u; worst_d = d; }
    ++n;
  }
  // exact differences x - m with a non-zero low part
  double worst2 = 0.0;
  unsigned s = 12345;
  for (int i = 0; i < 2000000; ++i) {
    s = s * 1103515245u + 12345u;
    float m = (float)((s >> 8) % 20000) / 97.0f - 60.0f;
    s = s * 1103515245u + 12345u;
    float x = m - (float)((s >> 8) % 1000000) * 1.19e-4f;
    float hi, lo;
    smx::two_diff(x, m, hi, lo);
    if (!(hi >= -120.0f)) continue;
    double ref = std::ldexp(std::exp((double)x - (double)m), 64);
    double u = ulp_err(smx::exp_biased64(hi, lo), ref);
    if (u > worst2) worst2 = u;
  }
  // factor of a merge, unscaled and in the 2^64 scale
  const float two64 = 18446744073709551616.0f;
  int bad_identity = (smx::exp_diff(-INFINITY, -INFINITY) != 1.0f) + (smx::exp_diff(3.0f, 3.0f) != 1.0f) +
                     (smx::exp_diff(-INFINITY, 2.0f) != 0.0f) +
                     (smx::exp_diff_b64(-INFINITY, -INFINITY) != two64) +
                     (smx::exp_diff_b64(3e38f, 3e38f) != two64) + (smx::exp_diff_b64(-INFINITY, 2.0f) != 0.0f) +
                     (smx::exp_diff_b64(-121.0f, 0.0f) != 0.0f) + (smx::exp_diff_b64(NAN, 0.0f) != 0.0f);
  // the scaled factor over pairs (a, b) of every magnitude whose difference
  // lies in [-120, 0], most of them below -87 (where the unscaled one is
  // subnormal): within an ulp of exp(a - b) 2^64, and equal to 2^64 times
  // the unscaled one wherever that is a normal number
  double worst_b64 = 0.0;
  int bad_scale = 0;
  for (int i = 0; i < 1000000; ++i) {
    s = s * 1103515245u + 12345u;
    const int ex = (int)((s >> 8) % 40) - 10;
    s = s * 1103515245u + 12345u;
    float b = std::ldexp((float)((s >> 8) & 0xFFFFFF) / 16777216.0f + 0.5f, ex);
    if (s & 1) b = -b;
    s = s * 1103515245u + 12345u;
    float a = b - (float)((s >> 8) % 1000000) * 1.2e-4f;
    const double d = (double)a - (double)b;  // exact for these magnitudes
    if (!(d >= -120.0) || !(a <= b)) continue;
    const float got = smx::exp_diff_b64(a, b);
    worst_b64 = std::fmax(worst_b64, ulp_err(got, std::ldexp(std::exp(d), 64)));
    const float un = smx::exp_diff(a, b);
    if (un >= 1.1754943508222875e-38f && (double)un != std::ldexp((double)got, -64)) ++bad_scale;
  }
  // bf16 rounding against a brute-force reference on a few patterns
  int bad_bf16 = 0;
  for (uint32_t u = 0; u < 0x7F800000u; u += 4093u) {
    float f = smx::u2f(u);
    uint32_t a = u >> 16, b = a + 1;
    double da = smx::u2f(a << 16);
    double db = b == 0x7F80u ? std::ldexp(1.0, 128) : (double)smx::u2f(b << 16);
    double dist_a = (double)f - da, dist_b = db - (double)f;
    uint32_t want = dist_a < dist_b ? a : (dist_b < dist_a ? b : ((a & 1) ? b : a));
    if (smx::bf16_rne(f) != want) ++bad_bf16;
  }
  // exp_dd_b64 / exp_dd_sum: every stride-th d in [-120, 0] against m = 0,
  // and seeded (x, m) pairs whose magnitudes run from 2^-30 to 2^100, x
  // within 120 below m; errors in ulps of the correctly rounded value
  struct Exp2Ref {
    float operator()(float t) const { return (float)std::exp2((double)t); }
  };
  double worst_dd = 0.0, worst_dd_sum = 0.0;
  for (uint64_t b = lo_bits; b <= hi_bits; b += stride) {
    float d = smx::u2f((uint32_t)b);
    double ref = std::exp((double)d);
    worst_dd = std::fmax(worst_dd, ulp_err(smx::exp_dd_b64(d, 0.0, Exp2Ref{}), std::ldexp(ref, 64)));
    if (d >= -87.0f) worst_dd_sum = std::fmax(worst_dd_sum, ulp_err(smx::exp_dd_sum(d, 0.0, Exp2Ref{}), ref));
  }
  for (int i = 0; i < 2000000; ++i) {
    s = s * 1103515245u + 12345u;
    const int ex = (int)((s >> 8) % 131) - 30;
    s = s * 1103515245u + 12345u;
    float m = std::ldexp((float)((s >> 8) & 0xFFFFFF) / 16777216.0f + 0.5f, ex);
    if (s & 1) m = -m;
    s = s * 1103515245u + 12345u;
    float x = m - (float)((s >> 8) % 1000000) * 1.2e-4f;  // fp32-rounded: x - m need not be that step
    if (!(x <= m)) continue;
    double d = (double)x - (double)m;  // exact for these magnitudes
    if (d < -120.0) continue;
    double ref = std::exp(d);
    worst_dd = std::fmax(worst_dd, ulp_err(smx::exp_dd_b64(x, (double)m, Exp2Ref{}), std::ldexp(ref, 64)));
    if (d >= -87.0) worst_dd_sum = std::fmax(worst_dd_sum, ulp_err(smx::exp_dd_sum(x, (double)m, Exp2Ref{}), ref));
  }
  // special cases: the maximum itself gives exactly 1 (2^64 scaled), at any
  // magnitude; lanes far below it (also where m - 160 rounds to m in fp32),
  // -inf and NaN give exactly 0
  int bad_dd = 0;
  const float big = 4294967296.0f;  // 2^32: m - 160 rounds back to m in fp32
  const float ms[] = {0.0f, 1.5f, -3.0f, big, -big, 1e30f, -3e38f, 3e38f};
  for (float m : ms) {
    bad_dd += smx::exp_dd_sum(m, (double)m, Exp2Ref{}) != 1.0f;
    bad_dd += smx::exp_dd_b64(m, (double)m, Exp2Ref{}) != 18446744073709551616.0f;
    bad_dd += smx::exp_dd_sum(-INFINITY, (double)m, Exp2Ref{}) != 0.0f;
    bad_dd += smx::exp_dd_b64(-INFINITY, (double)m, Exp2Ref{}) != 0.0f;
    bad_dd += smx::exp_dd_sum(NAN, (double)m, Exp2Ref{}) != 0.0f;
    bad_dd += smx::exp_dd_b64(NAN, (double)m, Exp2Ref{}) != 0.0f;
    const float below = std::nextafter(m, -INFINITY);  // one fp32 step below m
    const double gap = (double)below - (double)m;
    if (gap < -160.0) {
      bad_dd += smx::exp_dd_sum(below, (double)m, Exp2Ref{}) != 0.0f;
      bad_dd += smx::exp_dd_b64(below, (double)m, Exp2Ref{}) != 0.0f;
    }
  }
  bad_dd += smx::exp_dd_sum(big - 512.0f, (double)big, Exp2Ref{}) != 0.0f;
  std::printf("n=%ld max_ulp=%.4f at d=%.9g max_ulp_pair=%.4f bad_identity=%d bad_bf16=%d max_ulp_dd=%.4f "
              "max_ulp_dd_sum=%.4f bad_dd=%d max_ulp_diff_b64=%.4f bad_scale=%d\n",
              n, worst, worst_d, worst2, bad_identity, bad_bf16, worst_dd, worst_dd_sum, bad_dd, worst_b64, bad_scale);
  return 0;
}
