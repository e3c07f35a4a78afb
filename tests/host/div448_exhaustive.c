// Exhaustive host check of the write kernel's scale division (rkv_device.h,
// div448): for every fp32 x >= 2^-117 (below it the kernel divides), the product with RN(1/448)
// corrected once by its exact residual equals the correctly rounded x / 448.
// Exits 1 on any mismatch.
#include <math.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>
static float f(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
int main() {
  const float c = 1.0f / 448.0f;
  unsigned long long bad = 0, n = 0;
  for (uint32_t b = 0x05000000u; b < 0x7F800000u; ++b) {  // x >= 2^-117
    const float x = f(b);
    const float q0 = x * c;
    const float q1 = fmaf(fmaf(-q0, 448.0f, x), c, q0);
    const float ref = x / 448.0f;
    if (q1 != ref) { if (bad < 5) printf("x=%a q1=%a ref=%a\n", x, q1, ref); ++bad; }
    ++n;
  }
  printf("div448: %llu of %llu differ\n", bad, n);
  return bad != 0;
}
