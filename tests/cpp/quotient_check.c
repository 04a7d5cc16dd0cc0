/* Exhaustive host-side check of the encoder's division scheme (binary32, round to nearest).
 *
 * The GPU encoder computes q = x / d for the E2M1 rounding of each element as
 *     r = fl(1/d) (correctly rounded),  q0 = fl(x r),  e = -(fl(q0 d - x)) via FMA,
 *     q1 = fma(e, r, q0)
 * instead of a full IEEE division.  After one correction q1 is within half an ulp plus a
 * term of relative size ~2^-47 of x/d, so its E2M1 decision can only differ from that of
 * the IEEE quotient when x/d lies within a couple of ulps of one of the seven E2M1 rounding
 * thresholds.  This program enumerates every fp32 divisor mantissa (d in [1,2) and [2,4)),
 * every threshold, and every dividend within +-6 ulps of d*t, and compares both the
 * quotient and the E2M1 decision with IEEE division.  Scaling x and d by a common power of
 * two changes no rounding while everything stays normal, which the encoder guarantees by
 * using this path only for d in [2^-96, 2^100] and |x| <= 64 d.
 *
 * Exit status 0 iff no E2M1 decision differs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static inline float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E2M1 magnitude index of v >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to even, saturating */
static inline int e2m1_index(float v) {
  if (v <= 0.25f) return 0;
  if (v < 0.75f) return 1;
  if (v <= 1.25f) return 2;
  if (v < 1.75f) return 3;
  if (v <= 2.5f) return 4;
  if (v < 3.5f) return 5;
  if (v <= 5.0f) return 6;
  return 7;
}

int main(void) {
  static const float thresholds[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  long long checked = 0, decision_diff = 0, quotient_diff = 0;
#pragma omp parallel for reduction(+ : checked, decision_diff, quotient_diff) schedule(dynamic, 4096)
  for (long mant = 0; mant < (1L << 23); ++mant) {
    for (int e = 0; e < 2; ++e) {
      const float d = from_bits(((uint32_t)(127 + e) << 23) | (uint32_t)mant);
      volatile float one = 1.0f;
      const float r = one / d;
      for (int k = 0; k < 7; ++k) {
        const float c = d * thresholds[k];
        for (int o = -6; o <= 6; ++o) {
          const float x = from_bits(to_bits(c) + (uint32_t)o);
          const float q0 = x * r;
          const float err = -fmaf(q0, d, -x);
          const float q1 = fmaf(err, r, q0);
          const float ieee = x / d;
          checked++;
          quotient_diff += q1 != ieee;
          decision_diff += e2m1_index(q1) != e2m1_index(ieee);
        }
      }
    }
  }
  printf("checked %lld dividend/divisor pairs: %lld E2M1 decisions differ, %lld quotients differ\n",
         checked, decision_diff, quotient_diff);
  return decision_diff != 0;
}
