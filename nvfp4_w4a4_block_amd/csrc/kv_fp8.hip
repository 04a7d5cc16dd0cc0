// FP8 (E4M3FN) KV-cache codec with a calibrated per-tensor scale for gfx950.
//
// What is computed (calibrated FP8 key-value cache scales: paper abstract; "Quantizing All
// Layers Reveals Recurrent Memory Is Robust", "The Calibrated Cache That Ships for Free";
// "NVFP4 W4A4 Quantization Compresses 27B Hybrid Models", "Efficiency Gains and Serving
// Optimization"):
//   quantize:   byte = sign | E4M3_RNE_SAT(fl32(|x| / s)); +-inf -> +-448; NaN -> 0x7F
//   dequantize: y = fl32(E4M3(byte) * s); 0x7F / 0xFF -> NaN
// Memory-bound and elementwise: each thread takes 8 consecutive elements per iteration (one
// 16-byte bf16 load or two fp32 loads, one 8-byte store of bytes), grid-stride; the last
// n % 8 elements are done one per thread.
//
// Quantize, fast path (s in [2^-64, 2^64], decided once per launch): each element is clamped
// to +-fl32(440 s), divided with the one-correction quotient (reciprocal, product, one FMA
// residual step) and converted by the hardware E4M3 conversion (v_cvt_pk_fp8_f32).  The
// bytes equal those of the IEEE quotient under the software encoder:
//   - the clamp only moves values whose quotient rounds to 448 anyway (every quotient at or
//     above 432 does) to one that still does, and keeps infinities out of the division;
//   - for quotients in [2^-12, 1024] every intermediate of the one-correction quotient is
//     exactly a power-of-two scaling of a case in [1, 4), and an exhaustive host check over
//     every divisor significand finds its quotient equal to the IEEE one within six ulps of
//     every E4M3 decision point (decision points have significands 1 + m/16); elsewhere it
//     is a faithful rounding, which cannot cross a decision point;
//   - below 2^-12 both quotients encode to a signed zero byte;
//   - the hardware conversion rounds to nearest even with OCP E4M3FN subnormals and gives
//     the same byte as the software encoder for every fp32 value of magnitude at most 448.
// Eight elements of which any in the wave is NaN take the exact path (IEEE division and the
// software encoder), as does every element when s is outside the fast range (zero, tiny,
// huge, infinite or NaN scales).
// Dequantize uses the hardware E4M3 decode (v_cvt_pk_f32_fp8, exact, NaN for 0x7F / 0xFF)
// and one binary32 multiply.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kKvThreads = 256;

__device__ __forceinline__ uint32_t fp8_encode(float x, float s) {
  const float t = x / s;                                    // IEEE binary32 division
  const float a = __builtin_fabsf(t);
  if (a != a) return 0x7Fu;
  return e4m3_encode_rne_sat(a) | ((__float_as_uint(t) >> 24) & 0x80u);
}

// Operands of the fast quantize path: s, r = fl32(1 / s) and the clamp fl32(440 s).
struct FastQuotient {
  float s, r, lim;
};

__device__ __forceinline__ bool fast_scale(float s) { return s >= 0x1p-64f && s <= 0x1p64f; }

__device__ __forceinline__ float fast_quotient(float x, const FastQuotient& f) {
  return div_rn(__builtin_amdgcn_fmed3f(x, -f.lim, f.lim), f.s, f.r);
}

// Bytes of e[0..3] in one dword (element 0 in the low byte), fast path, non-NaN inputs.
__device__ __forceinline__ uint32_t fp8x4_fast(const float* e, const FastQuotient& f) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fast_quotient(e[0], f), fast_quotient(e[1], f), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fast_quotient(e[2], f), fast_quotient(e[3], f), (int)w, true);
}

__device__ __forceinline__ uint32_t fp8x4_exact(const float* e, float s) {
  return fp8_encode(e[0], s) | fp8_encode(e[1], s) << 8 | fp8_encode(e[2], s) << 16 | fp8_encode(e[3], s) << 24;
}

// fl32(E4M3(byte) * s) of the four bytes of w (byte 0 first): the hardware decode is exact
// and gives NaN for 0x7F / 0xFF, which the multiply keeps.
__device__ __forceinline__ void fp8x4_decode(int w, float s, float* e) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  e[0] = lo[0] * s;
  e[1] = lo[1] * s;
  e[2] = hi[0] * s;
  e[3] = hi[1] * s;
}

__device__ __forceinline__ void load8(const uint16_t* x, int64_t v, float (&e)[8]) {
  const uint4 w = reinterpret_cast<const uint4*>(x)[v];
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[2 * i] = __uint_as_float(a[i] << 16);
    e[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* x, int64_t v, float (&e)[8]) {
  const float4 a = reinterpret_cast<const float4*>(x)[2 * v];
  const float4 b = reinterpret_cast<const float4*>(x)[2 * v + 1];
  e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
  e[4] = b.x; e[5] = b.y; e[6] = b.z; e[7] = b.w;
}
__device__ __forceinline__ float load1(const uint16_t* x, int64_t i) { return __uint_as_float((uint32_t)x[i] << 16); }
__device__ __forceinline__ float load1(const float* x, int64_t i) { return x[i]; }

template <typename T>
__global__ __launch_bounds__(kKvThreads) void kv_quantize_kernel(const T* __restrict__ x, int64_t n,
                                                                 const float* __restrict__ scale,
                                                                 uint8_t* __restrict__ q) {
  const float s = scale[0];
  const int64_t nv = n / 8, stride = (int64_t)gridDim.x * kKvThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kKvThreads + threadIdx.x;
  if (fast_scale(s)) {
    const FastQuotient f{s, 1.0f / s, 440.0f * s};
    for (int64_t v = t0; v < nv; v += stride) {
      float e[8];
      load8(x, v, e);
      // Wave-wide NaN test (one compare per element, masks combined on the scalar unit):
      // a wave that meets a NaN takes the exact path for these eight elements.
      uint64_t nan = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) nan |= __builtin_amdgcn_ballot_w64(e[k] != e[k]);
      uint2 w;
      if (nan == 0) {
        w.x = fp8x4_fast(e, f);
        w.y = fp8x4_fast(e + 4, f);
      } else {
        w.x = fp8x4_exact(e, s);
        w.y = fp8x4_exact(e + 4, s);
      }
      reinterpret_cast<uint2*>(q)[v] = w;
    }
  } else {
    for (int64_t v = t0; v < nv; v += stride) {
      float e[8];
      load8(x, v, e);
      reinterpret_cast<uint2*>(q)[v] = make_uint2(fp8x4_exact(e, s), fp8x4_exact(e + 4, s));
    }
  }
  if (t0 < n - 8 * nv) q[8 * nv + t0] = (uint8_t)fp8_encode(load1(x, 8 * nv + t0), s);
}

template <bool BF16>
__global__ __launch_bounds__(kKvThreads) void kv_dequantize_kernel(const uint8_t* __restrict__ q, int64_t n,
                                                                   const float* __restrict__ scale,
                                                                   void* __restrict__ y) {
  const float s = scale[0];
  const int64_t nv = n / 8, stride = (int64_t)gridDim.x * kKvThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kKvThreads + threadIdx.x;
  for (int64_t v = t0; v < nv; v += stride) {
    const uint2 b = reinterpret_cast<const uint2*>(q)[v];
    float e[8];
    fp8x4_decode((int)b.x, s, e);
    fp8x4_decode((int)b.y, s, e + 4);
    if (BF16) {
      uint4 o;
      o.x = bf16_pair(e[0], e[1]);
      o.y = bf16_pair(e[2], e[3]);
      o.z = bf16_pair(e[4], e[5]);
      o.w = bf16_pair(e[6], e[7]);
      static_cast<uint4*>(y)[v] = o;
    } else {
      static_cast<float4*>(y)[2 * v] = make_float4(e[0], e[1], e[2], e[3]);
      static_cast<float4*>(y)[2 * v + 1] = make_float4(e[4], e[5], e[6], e[7]);
    }
  }
  if (t0 < n - 8 * nv) {
    float e[4];
    fp8x4_decode((int)q[8 * nv + t0], s, e);
    if (BF16)
      static_cast<uint16_t*>(y)[8 * nv + t0] = f32_to_bf16_rne(e[0]);
    else
      static_cast<float*>(y)[8 * nv + t0] = e[0];
  }
}

unsigned kv_grid(int64_t n) {
  const int64_t want = (n / 8 + kKvThreads - 1) / kKvThreads;
  const int64_t cap = 8 * 256;                  // enough resident workgroups to stream
  return (unsigned)(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace

int launch_kv_quantize(const void* x, int x_dtype, int64_t n, const float* scale, uint8_t* q, hipStream_t stream) {
  if (n == 0) return NVFP4_OK;
  if (x_dtype == NVFP4_BF16)
    kv_quantize_kernel<uint16_t><<<kv_grid(n), kKvThreads, 0, stream>>>(static_cast<const uint16_t*>(x), n, scale, q);
  else
    kv_quantize_kernel<float><<<kv_grid(n), kKvThreads, 0, stream>>>(static_cast<const float*>(x), n, scale, q);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int launch_kv_dequantize(const uint8_t* q, int64_t n, const float* scale, void* y, int y_dtype, hipStream_t stream) {
  if (n == 0) return NVFP4_OK;
  if (y_dtype == NVFP4_BF16)
    kv_dequantize_kernel<true><<<kv_grid(n), kKvThreads, 0, stream>>>(q, n, scale, y);
  else
    kv_dequantize_kernel<false><<<kv_grid(n), kKvThreads, 0, stream>>>(q, n, scale, y);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4
