// Host-side internals shared by the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

// Unsigned 32-bit division by a runtime constant with a multiply-high (round-up method of
// Granlund and Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDivU32 {
  uint32_t d, m, s1, s2;
};

inline FastDivU32 make_fastdiv(uint32_t d) {
  FastDivU32 f;
  f.d = d;
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < d) ++l;              // l = ceil(log2 d)
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, const FastDivU32& f) {
#ifdef __HIP_DEVICE_COMPILE__
  uint32_t t1 = __umulhi(f.m, n);
#else
  uint32_t t1 = (uint32_t)(((uint64_t)f.m * n) >> 32);
#endif
  return (t1 + ((n - t1) >> f.s1)) >> f.s2;
}

// Per-device facts (device.hip), set up once per device by the first call that launches work
// on it; safe to call from several host threads at once.
struct DeviceInfo {
  int cus;               // compute units
  void* quant_scratch;   // this device's copy of the quantizer's static scratch array
};

// The device `stream` belongs to (the current device for the null stream) and its facts.
int device_info(hipStream_t stream, DeviceInfo& info);

// Set-up steps of the kernel files, each run once per device with that device current.
int gemm_device_setup();                    // gemm.hip: LDS limits of the kernels that need more
int quantize_device_setup(void** scratch);  // quantize.hip: device address of the static scratch

// Quantize launchers (quantize.hip).  All validation is done by the caller.
int launch_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                    uint8_t* codes, uint8_t* scales, float* global_scale, int mode,
                    void* workspace, hipStream_t stream);
size_t quantize_workspace_bytes(int64_t rows, int64_t cols, int mode);
// Size of the static scratch array nvfp4_quantize_no_alloc uses in place of a workspace.
size_t quantize_scratch_bytes();

// GEMM launchers (gemm.hip).
struct SegmentTable {
  int32_t count;
  int32_t bound[NVFP4_MAX_SEGMENTS + 1];   // column offsets; bound[0] = 0, bound[count] = N
};

// NVFP4 output of the GEMM (quantized for the next linear layer under a given global
// scale): codes [M, N/2], scale bytes [M, N/16], both row-major and contiguous.
struct QuantOut {
  const float* global;
  uint8_t* codes;
  uint8_t* scales;
};

// Gated DeltaNet gates computed from the GEMM's fp32 output in the same launch: columns
// [n0, n0 + h) are the write-strength projection (beta = sigmoid(y)), columns [n0 + h, N) the
// decay projection (g = -exp(a_log[j]) * softplus(y + dt_bias[j]) for head j); g and beta are
// [M, h] fp32, row-major and contiguous; n0 + 2h == N.
struct GateOut {
  int32_t n0;
  int32_t h;
  const float* a_log;
  const float* dt_bias;
  float* g;
  float* beta;
};

// With qout set, y is unused and the result is written as NVFP4 instead; then N % 16 == 0 and
// the shape must be one the MFMA kernels take (NVFP4_ERR_UNSUPPORTED otherwise).  With gates
// set, y is written as usual and the gates as well; qout and gates are not combined.
// With swiglu, W's rows are gate/up pairs interleaved in groups of 16 (N % 32 == 0, w_globals =
// {gate, up}, seg unused) and the output is h = silu(gate) * up, [M, N/2]: in y (fp32 or bf16,
// pitch ldy) unless y is null, and as NVFP4 ([M, N/4] codes, [M, N/32] scales) when qout is set.
int launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                const float* a_global, int a_global_per_row, const uint8_t* w_codes,
                const uint8_t* w_scales, const float* w_globals, const SegmentTable& seg,
                void* y, int y_dtype, int64_t ldy, void* workspace, hipStream_t stream,
                const QuantOut* qout = nullptr, const GateOut* gates = nullptr, bool swiglu = false);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Batch-1 decode with the token's quantization fused in (per-row, which at one row is also
// per-tensor; or under the given global scale in a_global): one launch that writes the token's
// NVFP4 bytes to a_codes/a_scales (and a_global unless given) and Y = that token times W, the
// same bits as launch_quantize followed by launch_gemm wherever launch_gemm also takes the
// matrix-vector kernel.  bf16 input; NVFP4_ERR_UNSUPPORTED for a shape the kernel does not take
// (K % 64 != 0, K > 32768, or its LDS would not fit: about K <= 18432).
int launch_decode_linear(int64_t N, int64_t K, const uint16_t* x, bool given, uint8_t* a_codes, uint8_t* a_scales,
                         float* a_global, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                         void* y, int y_dtype, hipStream_t stream);

// MXFP4 operands (E2M1 codes [rows, K/2] as NVFP4, E8M0 scale bytes [rows, K/32]), the same
// tiling with scaled FP4 MFMAs; K % 256 == 0 and K < 2^24 (NVFP4_ERR_UNSUPPORTED otherwise).
int launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                   const float* a_global, int a_global_per_row, const uint8_t* w_codes, const uint8_t* w_scales,
                   const float* w_globals, const SegmentTable& seg, void* y, int y_dtype, int64_t ldy,
                   hipStream_t stream);

// Lossy NVFP4 -> MXFP4 re-encoding (mxfp4.hip); cols % 32 == 0, contiguous rows.
int launch_mx_reencode(int64_t rows, int64_t cols, const uint8_t* codes, const uint8_t* scales, uint8_t* mx_codes,
                       uint8_t* mx_scales, hipStream_t stream);

// FP8 KV-cache codec launchers (kv_fp8.hip).
int launch_kv_quantize(const void* x, int x_dtype, int64_t n, const float* scale, uint8_t* q, hipStream_t stream);
int launch_kv_dequantize(const uint8_t* q, int64_t n, const float* scale, void* y, int y_dtype, hipStream_t stream);

}  // namespace nvfp4
