/*
 * Exhaustive check of the oracle's binary32 -> binary16 round-to-nearest-even
 * converter against the x86 F16C instruction (vcvtps2ph, imm = round to
 * nearest), an independent hardware implementation of the same IEEE 754
 * conversion.  Every one of the 2^32 inputs is compared: bit-equal results,
 * except that a NaN input only has to give a NaN (payload handling is not
 * part of the rounding rule).  Also checks the exact widening of all 2^16
 * binary16 patterns against vcvtph2ps.  Test-suite helper; prints the count
 * of mismatches and exits non-zero if there is any.
 */
#include <immintrin.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../oracle/kda_oracle.h"

int main(void) {
  unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int64_t hi = 0; hi < 65536; ++hi) {
    for (uint32_t lo = 0; lo < 65536; ++lo) {
      const uint32_t u = ((uint32_t)hi << 16) | lo;
      float x;
      memcpy(&x, &u, 4);
      const uint16_t got = kdao_f32_to_f16_rne(x);
      const uint16_t ref = (uint16_t)_cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT);
      const int x_nan = (u & 0x7fffffffu) > 0x7f800000u;
      if (x_nan) {
        if (!((got & 0x7c00u) == 0x7c00u && (got & 0x3ffu))) ++bad;
      } else if (got != ref) {
        ++bad;
      }
    }
  }
  unsigned long long bad_w = 0;
  for (uint32_t h = 0; h < 65536; ++h) {
    const float got = kdao_f16_to_f32((uint16_t)h);
    const float ref = _cvtsh_ss((unsigned short)h);
    uint32_t gu, ru;
    memcpy(&gu, &got, 4);
    memcpy(&ru, &ref, 4);
    const int is_nan = ((h & 0x7c00u) == 0x7c00u) && (h & 0x3ffu);
    if (is_nan ? !(got != got) : gu != ru) ++bad_w;
  }
  printf("narrow_mismatches=%llu widen_mismatches=%llu\n", bad, bad_w);
  return (bad || bad_w) ? 1 : 0;
}
