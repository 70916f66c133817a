/* Pin for the oracle's E2M1 encoder: all 2^32 fp32 bit patterns (NaNs skipped) against
 * the closed form of round-to-nearest-even on the grid {0, .5, 1, 1.5, 2, 3, 4, 6}.
 * The midpoints between neighbouring grid values are .25 .75 1.25 1.75 2.5 3.5 5; the
 * magnitude code is the number of midpoints below |y|, where a midpoint whose upper
 * neighbour has an odd code (.25, 1.25, 2.5, 5) counts only when |y| is strictly above
 * it (the tie goes to the even code below) and the others count when |y| reaches them.
 * Linked with oracle/nvfp4_ref.c, whose oracle_e2m1_encode_f32 is under test. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

int oracle_e2m1_encode_f32(float y);

static int closed_form(float y) {
  float a = fabsf(y);
  int code = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return (signbit(y) ? 8 : 0) | code;
}

int main(void) {
  long long bad = 0;
  uint32_t first = 0;
  (void)oracle_e2m1_encode_f32(0.0f); /* initialise the grids before going parallel */
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (long long i = 0; i < (1LL << 32); ++i) {
    uint32_t bits = (uint32_t)i;
    float y;
    memcpy(&y, &bits, 4);
    if (isnan(y)) continue;
    if (oracle_e2m1_encode_f32(y) != closed_form(y)) {
      if (bad == 0) first = bits;
      ++bad;
    }
  }
  printf("mismatches %lld first 0x%08x\n", bad, first);
  return bad != 0;
}
