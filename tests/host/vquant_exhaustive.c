// Exhaustive host check of the write kernel's value-code rule (write_body.h,
// vquot_row / quant_v): for every bf16 amax in [1, 2) and every bf16 y with
// |y| <= amax, margins 1 and 1.5, the reciprocal exact or one ulp off either
// way, e4m3 of (Newton-corrected y/s) * (1 -/+ 2^-20 by the sign of the scale's
// rounding error) equals RNE e4m3 of the exact quotient.  Prints the counts;
// exits 1 on any mismatch.
#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>
static float bf(uint32_t h) { uint32_t b = h << 16; float x; memcpy(&x, &b, 4); return x; }
static uint32_t fb(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }
// e4m3fn RNE with saturation at 448 (value returned as double)
static double e4m3(double v) {
  double a = fabs(v);
  if (a >= 448.0) return copysign(448.0, v);
  int ex; frexp(a, &ex);  // a = f * 2^ex, f in [0.5,1)
  int e = ex - 1;          // a in [2^e, 2^(e+1))
  if (e < -6) e = -6;      // subnormal spacing 2^-9
  double step = ldexp(1.0, e - 3);
  double r = nearbyint(a / step) * step;  // ties to even (default mode)
  if (r > 448.0) r = 448.0;
  return copysign(r, v);
}
static float e4m3f(float v) { return (float)e4m3((double)v); }
int main() {
  const float margins[2] = {1.0f, 1.5f};
  unsigned long long n = 0, bad[3] = {0, 0, 0}, ties = 0;
  for (int mi = 0; mi < 2; ++mi)
  for (uint32_t ah = 0x3F80; ah < 0x4000; ++ah) {  // amax in [1, 2)
    const float A = bf(ah);
    const float Am = A * margins[mi];
    const float s = Am / 448.0f;
    const double es = fma((double)s, 448.0, -(double)Am);
    const float fct = es > 0 ? 1.0f - 0x1p-20f : (es < 0 ? 1.0f + 0x1p-20f : 1.0f);
    const float r0 = 1.0f / s;
    const float rr[3] = {r0, nextafterf(r0, 0.f), nextafterf(r0, INFINITY)};
    for (uint32_t yh = 0; yh < 0x7F80; ++yh) {
      const float ya = bf(yh);
      if (ya > A) break;
      for (int sg = 0; sg < 2; ++sg) {
        const float y = sg ? -ya : ya;
        const double ref = e4m3((double)y / (double)s);
        // exact tie check for the reference: y == m * s exactly for a midpoint m
        const double qd = (double)y / (double)s;
        { double a = fabs(qd); int ex; frexp(a, &ex); int e = ex - 1; if (e < -6) e = -6;
          double step = ldexp(1.0, e - 3); double k = a / step - floor(a / step);
          if (k == 0.5) ++ties; }
        for (int v = 0; v < 3; ++v) {
          const float r = rr[v];
          const float q0 = y * r;
          const float q = fmaf(fmaf(-q0, s, y), r, q0) * fct;
          const float qc = fminf(fmaxf(q, -448.f), 448.f);
          if ((double)e4m3f(qc) != ref) { if (bad[v] < 4) printf("m %g A %a y %a v %d got %g ref %g q %a\n", margins[mi], A, y, v, e4m3f(qc), ref, q); ++bad[v]; }
        }
        ++n;
      }
    }
  }
  printf("pairs %llu exact-tie quotients %llu  mismatches r=RN %llu r-1ulp %llu r+1ulp %llu\n", n, ties, bad[0], bad[1], bad[2]);
  return (bad[0] | bad[1] | bad[2]) != 0;
}
