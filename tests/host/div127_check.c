/* Host-side check of the q8_K block-scale arithmetic the GPU kernels use
 * (q8k_div127 in bit_quantized_matvec_amd/csrc/q8k_block.h): for c = fl(1/127),
 * p = fl(a c), r = fma(-p, 127, a), d = fma(r, c, p) must equal the IEEE
 * quotient fl(a / 127).  Checked for every fp32 significand at the exponents
 * given on the command line (biased, 1..254); within the normal range the
 * outcome depends on the significand alone.  Prints the mismatch count. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int main(int argc, char **argv) {
  const float c = 1.0f / 127.0f;
  long bad = 0, n = 0;
  for (int i = 1; i < argc; ++i) {
    const uint32_t e = (uint32_t)atoi(argv[i]);
    for (uint32_t m = 0; m < (1u << 23); ++m) {
      const uint32_t u = (e << 23) | m;
      float a;
      memcpy(&a, &u, 4);
      const float want = a / 127.0f;
      const float p = a * c;
      const float r = fmaf(-p, 127.0f, a);
      const float got = fmaf(r, c, p);
      ++n;
      if (memcmp(&got, &want, 4) != 0) ++bad;
    }
  }
  printf("%ld %ld\n", n, bad);
  return 0;
}
