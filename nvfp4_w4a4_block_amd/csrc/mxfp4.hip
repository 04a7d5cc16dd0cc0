// Lossy re-encoding of NVFP4 tensors to MXFP4 for gfx950's scaled FP4 matrix instructions.
//
// What is computed.  NVFP4 holds E2M1 element codes with one E4M3 scale per 16-element block
// ("NVFP4 W4A4 Quantization Compresses 27B Hybrid Models", section "Challenging the
// Recurrence Fragility Assumption"); MXFP4 holds E2M1 codes with one E8M0 (power of two)
// scale per 32-element block (OCP Microscaling (MX) specification v1.0, which also gives the
// scale rule used here).  Each 32-element block (two NVFP4 blocks) of a row is re-encoded from
// its exact NVFP4 values v = E2M1 * E4M3, the tensor's global scale staying aside as a
// multiplier:
//   e = floor(log2(max |v|)) - 2,  E8M0 byte = e + 127,
//   magnitude = E2M1_RNE_SAT(|v| / 2^e)   (ties to even, above 6 saturating to 6),
//   sign bit copied from the NVFP4 code; a block of zeros gets byte 0 and magnitude 0.
// The E4M3 mantissa of each NVFP4 block scale is lost, and the smaller block of the pair is
// rounded on the larger one's grid: the re-encoding is lossy by design.
//
// Design: memory-bound and elementwise over blocks.  Codes and scale bytes are row-major and
// contiguous, so block b of the flattened tensor is 16 bytes of codes at 16 b and two E4M3
// bytes at 2 b, and its outputs are 16 bytes at 16 b and one E8M0 byte at b.  One thread per
// block, grid-stride.  Every value step is exact in fp32 (E2M1 * E4M3 has at most 6
// significant bits; scaling by 2^-e is exact), and the final rounding is the hardware E2M1
// conversion (round to nearest even, saturating).
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kMxThreads = 256;

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// E2M1 magnitude of a 3-bit index (exact fp32): 0, 0.5, then (1 + m/2) * 2^(e-1).
__device__ __forceinline__ float e2m1_magnitude(uint32_t i) {
  if (i < 2) return 0.5f * (float)i;
  return __uint_as_float(((126u + (i >> 1)) << 23) | ((i & 1u) << 22));
}

// Largest 3-bit magnitude index among the 8 codes of a dword.
__device__ __forceinline__ uint32_t max_magnitude(uint32_t w) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, (w >> (4 * k)) & 7u);
  return m;
}

// Re-encode the 8 codes of one dword: magnitudes times t (= E4M3 scale * 2^-e, exact), rounded
// to E2M1 by the hardware conversion, then the original sign bits.
__device__ __forceinline__ uint32_t reencode8(uint32_t w, float t) {
  const uint32_t mag = w & 0x77777777u;
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2_t v = b == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(mag, 1.0f, 0)
                      : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(mag, 1.0f, 1)
                      : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(mag, 1.0f, 2)
                               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(mag, 1.0f, 3);
    const float q0 = v[0] * t, q1 = v[1] * t;
    out = b == 0   ? __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, q0, q1, 1.0f, 0)
          : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, q0, q1, 1.0f, 1)
          : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, q0, q1, 1.0f, 2)
                   : __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, q0, q1, 1.0f, 3);
  }
  return out | (w & 0x88888888u);
}

__global__ __launch_bounds__(kMxThreads) void mx_reencode_kernel(const uint4* codes, const uint16_t* scales,
                                                                 uint4* mx_codes, uint8_t* mx_scales,
                                                                 int64_t nblocks) {
  for (int64_t b = (int64_t)blockIdx.x * kMxThreads + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * kMxThreads) {
    const uint4 c = codes[b];
    const uint32_t s2 = scales[b];
    const float s0 = e4m3_decode(s2 & 0xFFu), s1 = e4m3_decode(s2 >> 8);
    const float amax = __builtin_fmaxf(e2m1_magnitude(max(max_magnitude(c.x), max_magnitude(c.y))) * s0,
                                       e2m1_magnitude(max(max_magnitude(c.z), max_magnitude(c.w))) * s1);
    uint32_t byte = 0;
    uint4 out = make_uint4(c.x & 0x88888888u, c.y & 0x88888888u, c.z & 0x88888888u, c.w & 0x88888888u);
    if (amax != 0.0f) {
      // amax >= 2^-10 is a normal fp32: floor(log2(amax)) = eb - 127, so e = eb - 129.
      const uint32_t eb = (__float_as_uint(amax) >> 23) & 0xFFu;
      byte = eb - 2u;
      const float inv = __uint_as_float((256u - eb) << 23);       // 2^-e
      const float t0 = s0 * inv, t1 = s1 * inv;
      out = make_uint4(reencode8(c.x, t0), reencode8(c.y, t0), reencode8(c.z, t1), reencode8(c.w, t1));
    }
    mx_codes[b] = out;
    mx_scales[b] = (uint8_t)byte;
  }
}

}  // namespace

int launch_mx_reencode(int64_t rows, int64_t cols, const uint8_t* codes, const uint8_t* scales, uint8_t* mx_codes,
                       uint8_t* mx_scales, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return NVFP4_OK;
  const int64_t want = (nblocks + kMxThreads - 1) / kMxThreads;
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  mx_reencode_kernel<<<grid, kMxThreads, 0, stream>>>(reinterpret_cast<const uint4*>(codes),
                                                       reinterpret_cast<const uint16_t*>(scales),
                                                       reinterpret_cast<uint4*>(mx_codes), mx_scales, nblocks);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4
