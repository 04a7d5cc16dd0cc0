// Calibration kernels for the measurement script (libnvfp4_calib.so, not the library's path):
// what a plain streaming read, a plain copy and a loop of nothing but fp16 MFMAs reach on this
// GPU, so that the hot path's roofline fractions can be read against measured ceilings as
// well as against the published peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense fp16).
//
//   nvfp4_calib_read(p, bytes, sink, stream)    reads `bytes` (a multiple of 16) once
//   nvfp4_calib_copy(src, dst, bytes, stream)   reads and writes `bytes` once
//   nvfp4_calib_mfma(waves, iters, sink, stream) `waves` wavefronts, each issuing 4 * iters
//                                                v_mfma_f32_32x32x16_f16 (32768 flops each)
// `sink` is a device buffer of at least 4 bytes; it is written only if a computed value equals
// a constant no input produces, which keeps every load and MFMA alive without adding traffic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;       // independent 16-byte loads per thread per iteration
constexpr uint32_t kNever = 0x9E3779B9u;

__global__ __launch_bounds__(kThreads) void calib_read_kernel(const uint4* __restrict__ p, int64_t n,
                                                              uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kNever) sink[0] = acc;
}

__global__ __launch_bounds__(kThreads) void calib_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                              int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(kThreads) void calib_mfma_kernel(int iters, uint32_t* __restrict__ sink) {
  // four independent accumulator chains, each with operands of its own (no two MFMAs alike)
  half8_t a0, a1, a2, a3, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = (_Float16)(float)((threadIdx.x + i) & 7);
    a1[i] = (_Float16)(float)((threadIdx.x + i + 1) & 7);
    a2[i] = (_Float16)(float)((threadIdx.x + i + 2) & 7);
    a3[i] = (_Float16)(float)((threadIdx.x + i + 3) & 7);
    b[i] = (_Float16)(float)((threadIdx.x * 3 + i) & 7);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a2, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a3, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (__float_as_uint(s) == kNever) sink[0] = kNever;
}

unsigned read_grid(int64_t n) {
  // one iteration of kUnroll loads per thread when the buffer allows, as a single pass would
  const int64_t per_wg = (int64_t)kThreads * kUnroll;
  int64_t g = (n + per_wg - 1) / per_wg;
  return (unsigned)(g < 1 ? 1 : g > (1 << 20) ? (1 << 20) : g);
}

}  // namespace

extern "C" {

int nvfp4_calib_read(const void* p, int64_t bytes, void* sink, void* stream) {
  if (!p || !sink || bytes <= 0 || bytes % 16 != 0) return 1;
  const int64_t n = bytes / 16;
  calib_read_kernel<<<read_grid(n), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(p), n, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int nvfp4_calib_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 != 0) return 1;
  const int64_t n = bytes / 16;
  calib_copy_kernel<<<read_grid(n), kThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int nvfp4_calib_mfma(int waves, int iters, void* sink, void* stream) {
  if (!sink || waves <= 0 || waves % 4 != 0 || iters <= 0) return 1;
  calib_mfma_kernel<<<waves / 4, kThreads, 0, static_cast<hipStream_t>(stream)>>>(iters,
                                                                                  static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
