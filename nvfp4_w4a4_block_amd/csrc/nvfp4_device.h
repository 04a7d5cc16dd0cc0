// Device helpers for NVFP4 on gfx950: E4M3 block-scale encode/decode, the exact binary32
// quotient used by the encoder, and exact dequantization of packed E2M1 codes to fp16.
//
// Format: E2M1 element codes with one E4M3 scale per 16-element block ("NVFP4 W4A4
// Quantization Compresses 27B Hybrid Models", section "Challenging the Recurrence
// Fragility Assumption"), under an FP32 per-module global scale (the global-scale mismatch
// in the paper abstract presupposes one).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kGlobalDivisor = 2688.0f;   // largest E2M1 (6) times largest E4M3 (448)

// E4M3FN byte of the value nearest to t (t >= 0, not NaN), ties to the even byte, t above
// 448 saturating to 448 (0x7E).  Subnormal range (t < 2^-6) has spacing 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float t) {
  if (!(t < 464.0f)) return 0x7Eu;                 // 464 is the 448/480 midpoint -> 448
  if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);   // 0..8, exact scaling
  uint32_t u = __float_as_uint(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);                // round mantissa to 3 bits, ties even
  uint32_t b = ((u >> 20) & 0x7FFu) - (120u << 3); // rebias exponent 127 -> 7
  return b > 0x7Eu ? 0x7Eu : b;
}

// Value of an E4M3FN byte in [0, 0x7E] as fp32 (exact).
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  uint32_t e = b >> 3, m = b & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// fl32(x / d) for d in [2^-96, 2^100] and |x| <= 64 d, given r = fl32(1 / d): the product
// x r and one FMA residual correction (Markstein's correction step).  After the correction
// the quotient is within half an ulp plus a term of relative size ~2^-47 of x / d, so its
// E2M1 rounding can differ from that of the IEEE quotient only within a couple of ulps of
// an E2M1 rounding threshold; an exhaustive host-side check over every divisor mantissa
// near every threshold finds no difference.  The residual is formed as -(q d - x) rather
// than x - q d so that an exact zero residual keeps the sign of x (x = -0 gives -0).
__device__ __forceinline__ float div_rn(float x, float d, float r) {
  const float q = x * r;
  const float e = -__builtin_fmaf(q, d, -x);
  return __builtin_fmaf(e, r, q);
}

// 16 B of input as fp32 values.
__device__ __forceinline__ void widen(const uint4& w, float* v, const uint16_t*) {
  uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(a[i] << 16);
    v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void widen(const uint4& w, float* v, const float*) {
  v[0] = __uint_as_float(w.x);
  v[1] = __uint_as_float(w.y);
  v[2] = __uint_as_float(w.z);
  v[3] = __uint_as_float(w.w);
}

// Largest |x| bit pattern of 16 B of input, as an fp32 bit pattern.  Integer max of the
// magnitude bits orders NaN above +inf above every finite value, so NaN propagates.
__device__ __forceinline__ uint32_t max_abs_bits(const uint4& w, const uint16_t*) {
  uint32_t m = 0;
  uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = (a[i] & 0x7FFFu), hi = (a[i] >> 16) & 0x7FFFu;
    m = max(m, max(lo, hi));
  }
  return m << 16;
}
__device__ __forceinline__ uint32_t max_abs_bits(const uint4& w, const float*) {
  return max(max(w.x & 0x7FFFFFFFu, w.y & 0x7FFFFFFFu), max(w.z & 0x7FFFFFFFu, w.w & 0x7FFFFFFFu));
}

// Encode one 16-element block (values v[0..15] as fp32) under global scale sg.
// Outputs the E4M3 scale byte and the 16 codes packed into two dwords (element 2i in the
// low nibble of byte i).  Arithmetic: binary32, round to nearest even, no contraction.
__device__ __forceinline__ void encode_block(const float (&v)[16], float sg, uint32_t& scale_byte,
                                             uint32_t& lo, uint32_t& hi) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
  uint32_t s = 0;
  if (sg != 0.0f) {
    float den = 6.0f * sg;
    float t = a / den;                         // IEEE division (correctly rounded)
    s = (t == t) ? e4m3_encode_rne_sat(t) : 0u;
  }
  float d = e4m3_decode(s) * sg;
  float q[16];
  bool fast = d >= 0x1p-96f && d <= 0x1p100f && a <= 64.0f * d;
  if (fast) {
    float r = 1.0f / d;
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = div_rn(v[i], d, r);
  } else if (d == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = __builtin_copysignf(0.0f, v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = v[i] / d;
  }
  // Hardware E2M1 conversion: round to nearest even, saturating at 6, sign kept (scale
  // operand 1.0 leaves the value unscaled).  Operand a goes to the low nibble.
  uint32_t w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[0], q[1], 1.0f, 0);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[2], q[3], 1.0f, 1);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[4], q[5], 1.0f, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, q[6], q[7], 1.0f, 3);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[8], q[9], 1.0f, 0);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[10], q[11], 1.0f, 1);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[12], q[13], 1.0f, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, q[14], q[15], 1.0f, 3);
  scale_byte = s;
  lo = w0;
  hi = w1;
}

// fp16 pair (E4M3(s) * 2^-8, E4M3(s) * 2^-8) from a scale byte: the E4M3 bit pattern shifted
// into the fp16 exponent/mantissa fields has the same value divided by 2^8 (bias 15 vs 7),
// subnormals included.  Exact.
__device__ __forceinline__ half2_t scale_pair_f16(uint32_t s_byte) {
  uint32_t bits = (s_byte << 7) | (s_byte << 23);
  return __builtin_bit_cast(half2_t, bits);
}

// Dequantize the 8 codes of one dword (element 2i in the low nibble of byte i) to fp16,
// multiplied by the block scale.  The conversion scales by 2^8 (only the exponent of its
// scale operand is used) and the fp16 multiply by E4M3 * 2^-8, so every product is the
// exact E2M1 * E4M3 value (at most 6 significant bits, range [2^-10, 2688]).
__device__ __forceinline__ half8_t dequant8_f16(uint32_t codes, half2_t sc) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0);
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1);
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2);
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3);
  p0 *= sc;
  p1 *= sc;
  p2 *= sc;
  p3 *= sc;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Round fp32 to bfloat16 bits, nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values -> packed bf16 (lo in the low half) by the hardware conversion: round to
// nearest even, NaN kept NaN with the quiet bit set.  Gives the same bits as f32_to_bf16_rne
// for every fp32 input.
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

}  // namespace nvfp4
