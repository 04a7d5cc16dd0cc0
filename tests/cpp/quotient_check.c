/* Exhaustive host-side check of the encoders' division scheme (binary32, round to nearest).
 *
 * The GPU encoders compute q = x / d as
 *     r = fl(1/d) (correctly rounded),  q0 = fl(x r),  e = -(fl(q0 d - x)) via FMA,
 *     q1 = fma(e, r, q0)
 * instead of a full IEEE division.  After one correction q1 is within half an ulp plus a
 * term of relative size ~2^-46 of x/d (a faithful rounding), so a rounding decision taken
 * on q1 can only differ from the one taken on the IEEE quotient when x/d lies within about
 * one ulp of a decision point.  This program enumerates every fp32 divisor mantissa (d in
 * [1,2) and [2,4)), every decision point, and every dividend within +-6 ulps of d*t, and
 * compares both the quotient and the decision with IEEE division.  Scaling x and d by a
 * common power of two changes no rounding while every intermediate stays exactly
 * representable, which each encoder's fast-path guard ensures.
 *
 * Mode "e2m1" (default): the seven E2M1 rounding thresholds {0.25, 0.75, 1.25, 1.75, 2.5,
 * 3.5, 5}; the decision is the E2M1 magnitude index.
 * Mode "e4m3": every E4M3FN decision point has a significand of the form 1 + m/16 (the
 * midpoints between normal neighbours are (1 + (2j+1)/16) 2^E, those of the subnormal
 * range (2k+1) 2^-10 reduce to 1 + (even m)/16), so the sixteen values t = 1 + m/16,
 * m = 0..15, cover every decision point up to a power of two; the decision is which side
 * of t the quotient falls on (below, equal, above), which fixes the E4M3 rounding there.
 *
 * Exit status 0 iff no decision differs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static inline float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E2M1 magnitude index of v >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to even, saturating */
static inline int e2m1_index(float v, float t) {
  (void)t;
  if (v <= 0.25f) return 0;
  if (v < 0.75f) return 1;
  if (v <= 1.25f) return 2;
  if (v < 1.75f) return 3;
  if (v <= 2.5f) return 4;
  if (v < 3.5f) return 5;
  if (v <= 5.0f) return 6;
  return 7;
}

/* Side of the decision point t that v falls on. */
static inline int side(float v, float t) { return (v > t) - (v < t); }

int main(int argc, char** argv) {
  static const float e2m1_points[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  float e4m3_points[16];
  for (int m = 0; m < 16; ++m) e4m3_points[m] = 1.0f + (float)m / 16.0f;
  const int e4m3 = argc > 1 && strcmp(argv[1], "e4m3") == 0;
  const float* points = e4m3 ? e4m3_points : e2m1_points;
  const int npoints = e4m3 ? 16 : 7;
  int (*decide)(float, float) = e4m3 ? side : e2m1_index;
  long long checked = 0, decision_diff = 0, quotient_diff = 0;
#pragma omp parallel for reduction(+ : checked, decision_diff, quotient_diff) schedule(dynamic, 4096)
  for (long mant = 0; mant < (1L << 23); ++mant) {
    for (int e = 0; e < 2; ++e) {
      const float d = from_bits(((uint32_t)(127 + e) << 23) | (uint32_t)mant);
      volatile float one = 1.0f;
      const float r = one / d;
      for (int k = 0; k < npoints; ++k) {
        const float t = points[k];
        const float c = d * t;
        for (int o = -6; o <= 6; ++o) {
          const float x = from_bits(to_bits(c) + (uint32_t)o);
          const float q0 = x * r;
          const float err = -fmaf(q0, d, -x);
          const float q1 = fmaf(err, r, q0);
          const float ieee = x / d;
          checked++;
          quotient_diff += q1 != ieee;
          decision_diff += decide(q1, t) != decide(ieee, t);
        }
      }
    }
  }
  printf("checked %lld dividend/divisor pairs: %lld %s decisions differ, %lld quotients differ\n",
         checked, decision_diff, e4m3 ? "E4M3" : "E2M1", quotient_diff);
  return decision_diff != 0;
}
