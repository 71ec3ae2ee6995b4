/*
 * Exhaustive pin of the oracle's number converters (test infrastructure; CPU only).
 *
 * Every one of the 2^32 binary32 bit patterns is widened to double (exact) and rounded
 * by the oracle's converters to bfloat16 and binary16.  The expected result comes from
 * sources other than the oracle:
 *   - binary16: the x86 F16C conversion instruction (vcvtps2ph) with round-to-nearest-even,
 *     the IEEE 754 conversion done in hardware;
 *   - bfloat16: round-to-nearest-even on the integer bit pattern (bfloat16 is the upper
 *     half of binary32: add 0x7fff plus the lowest kept bit, then drop the low 16 bits;
 *     a carry out of the fraction increments the exponent, reaching infinity at the top).
 * NaNs must stay NaNs of the same sign.  Prints the number of mismatches per format and
 * the lowest mismatching pattern of each; exit status 0 when there are none.
 */
#include <immintrin.h>
#include <stdio.h>

#include "../../oracle/emb_oracle.c"

static int is_nan16(uint16_t h, int expo_bits) {
  if (expo_bits == 5) return (h & 0x7c00) == 0x7c00 && (h & 0x03ff) != 0;
  return (h & 0x7f80) == 0x7f80 && (h & 0x007f) != 0;
}

int main(void) {
  long long bad_bf16 = 0, bad_f16 = 0;
  uint32_t first_bf16 = 0, first_f16 = 0;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad_bf16, bad_f16)
  for (long long i = 0; i < (1LL << 32); ++i) {
    const uint32_t u = (uint32_t)i;
    float f;
    memcpy(&f, &u, sizeof f);
    const double x = (double)f;
    const int nan = (u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0;
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);

    const uint16_t got_b = double_to_bf16_bits(x);
    int ok_b;
    if (nan) {
      ok_b = is_nan16(got_b, 8) && (got_b & 0x8000u) == sign;
    } else {
      const uint32_t ref = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
      ok_b = got_b == (uint16_t)ref;
    }
    if (!ok_b) {
#pragma omp critical
      if (first_bf16 == 0 || u < first_bf16) first_bf16 = u;
      ++bad_bf16;
    }

    const uint16_t got_h = double_to_f16_bits(x);
    const uint16_t ref_h = (uint16_t)_cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT);
    const int ok_h = nan ? (is_nan16(got_h, 5) && (got_h & 0x8000u) == sign) : got_h == ref_h;
    if (!ok_h) {
#pragma omp critical
      if (first_f16 == 0 || u < first_f16) first_f16 = u;
      ++bad_f16;
    }
  }
  printf("bf16 mismatches %lld (first 0x%08x)\n", bad_bf16, first_bf16);
  printf("f16 mismatches %lld (first 0x%08x)\n", bad_f16, first_f16);
  return (bad_bf16 || bad_f16) ? 1 : 0;
}
