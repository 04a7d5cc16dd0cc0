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
// n % 8 elements are done one per thread.  The quotient is the IEEE binary32 division and the
// E4M3 rounding is the encoder of the NVFP4 block scales (round to nearest even, saturating).
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

__device__ __forceinline__ float fp8_decode(uint32_t b, float s) {
  const uint32_t m = b & 0x7Fu;
  if (m == 0x7Fu) return __builtin_nanf("");
  const float v = e4m3_decode(m) * s;
  return (b & 0x80u) ? -v : v;
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
  for (int64_t v = t0; v < nv; v += stride) {
    float e[8];
    load8(x, v, e);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= fp8_encode(e[k], s) << (8 * k);
      hi |= fp8_encode(e[k + 4], s) << (8 * k);
    }
    reinterpret_cast<uint2*>(q)[v] = make_uint2(lo, hi);
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
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      e[k] = fp8_decode((b.x >> (8 * k)) & 0xFFu, s);
      e[k + 4] = fp8_decode((b.y >> (8 * k)) & 0xFFu, s);
    }
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
    const float v = fp8_decode(q[8 * nv + t0], s);
    if (BF16)
      static_cast<uint16_t*>(y)[8 * nv + t0] = f32_to_bf16_rne(v);
    else
      static_cast<float*>(y)[8 * nv + t0] = v;
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
