// Host build of the kernels' scalar arithmetic (smx_math.hpp), checked
// against libm's double-precision exp. Prints one line of results.
//   check_smx_math <stride>
// walks every stride-th fp32 value d in [-120, 0] with dl = 0, plus a seeded
// set of (dh, dl) pairs formed as exact differences of two fp32 values.
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
  // factor of a merge
  int bad_identity = (smx::exp_diff(-INFINITY, -INFINITY) != 1.0f) + (smx::exp_diff(3.0f, 3.0f) != 1.0f) +
                     (smx::exp_diff(-INFINITY, 2.0f) != 0.0f);
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
  std::printf("n=%ld max_ulp=%.4f at d=%.9g max_ulp_pair=%.4f bad_identity=%d bad_bf16=%d\n", n, worst,
              worst_d, worst2, bad_identity, bad_bf16);
  return 0;
}
