// NVFP4 quantization kernels for gfx950.
//
// Steps, per "Why Gated DeltaNet Survives 4-Bit Quantization" ("The deep dive": four-bit
// values, one shared scale per sixteen-element block) and "NVFP4 W4A4 Quantization
// Compresses 27B Hybrid Models" (section "Challenging the Recurrence Fragility
// Assumption": E2M1 values, E4M3 block scale):
//   global scale  s_g = fl32(max|x| / 2688)  (per tensor or per row; or given)
//   block scale   s_j = E4M3_RNE_SAT(fl32(a_j / fl32(6 s_g))),  a_j = max |x| of the block
//   element       code = sign | E2M1_RNE_SAT(fl32(x / fl32(E4M3(s_j) s_g)))
//
// Memory-bound design: one lane encodes one 16-element block (32 B of bf16 in, 8 B of codes
// and 1 B of scale out), so a wavefront streams 2 KB of contiguous input per block row.  The
// per-tensor global scale needs a grid-wide max before the first block can be encoded:
// pass 1 writes one NaN-propagating partial max per workgroup, and every workgroup of pass
// 2 reduces those few partials itself, so no atomics, counters or zero-initialised
// workspace are needed and the result is deterministic.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kWideThreads = 1024;       // per-row workgroups when there are fewer rows than CUs
constexpr int kMaxPartials = 1024;        // pass-1 workgroups (4 partials per pass-2 thread)

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Workgroup max of one value per thread (NT threads); the result is valid in every thread.
template <int NT = kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[NT / 64];
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = max(r, red[i]);
  __syncthreads();
  return r;
}

template <typename T>
constexpr int kElemsPer16B = 16 / sizeof(T);

// Pass 1 of the per-tensor mode: one partial max (fp32 magnitude bits) per workgroup.
// Contiguous input is read as a flat array of 16 B chunks, four independent loads per
// thread per iteration; otherwise workgroups stride over rows and threads over a row.
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const T* __restrict__ x, int64_t rows,
                                                                 int64_t cols, int64_t ldx,
                                                                 uint32_t* __restrict__ partial) {
  const int64_t chunks = cols / kElemsPer16B<T>;
  uint32_t m = 0;
  if (ldx == cols) {
    // With a grid that is a multiple of 8, the workgroups of XCD x (blockIdx % 8, dispatch is
    // round-robin over the 8 XCDs) read the x-th eighth of the tensor, in increasing address
    // order; the encoder reads the same eighth on the same XCD in decreasing order, so its
    // first reads hit what this pass left in that XCD's L2.
    const uint4* p = reinterpret_cast<const uint4*>(x);
    const int64_t total = rows * chunks;
    int64_t lo = 0, hi = total, stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if ((gridDim.x & 7) == 0) {
      const int xcd = blockIdx.x & 7;
      lo = total * xcd / 8;
      hi = total * (xcd + 1) / 8;
      stride = (int64_t)(gridDim.x >> 3) * kThreads;
      i = lo + (int64_t)(blockIdx.x >> 3) * kThreads + threadIdx.x;
    }
    for (; i + 3 * stride < hi; i += 4 * stride) {
      const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
      m = max(m, max(max(max_abs_bits(a, x), max_abs_bits(b, x)), max(max_abs_bits(c, x), max_abs_bits(d, x))));
    }
    for (; i < hi; i += stride) m = max(m, max_abs_bits(p[i], x));
  } else {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
      const uint4* row = reinterpret_cast<const uint4*>(x + r * ldx);
      for (int64_t c = threadIdx.x; c < chunks; c += kThreads) m = max(m, max_abs_bits(row[c], x));
    }
  }
  m = block_max_u32(m);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Per-row global scales: one workgroup per row (strided), s_g[r] = fl32(amax_r / 2688).
template <typename T>
__global__ __launch_bounds__(kThreads) void row_scale_kernel(const T* __restrict__ x, int64_t rows,
                                                              int64_t cols, int64_t ldx,
                                                              float* __restrict__ sg_out) {
  const int64_t chunks = cols / kElemsPer16B<T>;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint4* row = reinterpret_cast<const uint4*>(x + r * ldx);
    uint32_t m = 0;
    for (int64_t c = threadIdx.x; c < chunks; c += kThreads) m = max(m, max_abs_bits(row[c], x));
    m = block_max_u32(m);
    if (threadIdx.x == 0) sg_out[r] = __uint_as_float(m) / kGlobalDivisor;
  }
}

// Per-row mode in one pass: one workgroup of NT threads per row (strided over rows) keeps the
// row's blocks in registers (up to MAXB per thread), reduces the row max, writes s_g[r] and
// encodes.  Few rows (decode) take 1024-thread workgroups, so each thread has one or two
// blocks to load and encode; many rows take 256-thread workgroups, several per CU.
template <typename T, int MAXB, int NT = kThreads>
__global__ __launch_bounds__(NT) void row_quant_kernel(const T* __restrict__ x, int64_t rows, uint32_t bpr,
                                                              int64_t ldx, uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales,
                                                              float* __restrict__ sg_out) {
  constexpr int NC = 16 / kElemsPer16B<T>;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const T* row = x + r * ldx;
    uint4 w[MAXB][NC];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < MAXB; ++j) {
      const uint32_t b = threadIdx.x + j * NT;
      if (b < bpr) {
        const uint4* p = reinterpret_cast<const uint4*>(row + (int64_t)b * 16);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          w[j][c] = p[c];
          m = max(m, max_abs_bits(w[j][c], x));
        }
      }
    }
    m = block_max_u32<NT>(m);
    const float sg = __uint_as_float(m) / kGlobalDivisor;
    if (threadIdx.x == 0) sg_out[r] = sg;
#pragma unroll
    for (int j = 0; j < MAXB; ++j) {
      const uint32_t b = threadIdx.x + j * NT;
      if (b < bpr) {
        float v[16];
#pragma unroll
        for (int c = 0; c < NC; ++c) widen(w[j][c], v + c * kElemsPer16B<T>, x);
        uint32_t sb, lo, hi;
        encode_block(v, sg, sb, lo, hi);
        const int64_t i = r * (int64_t)bpr + b;
        reinterpret_cast<uint2*>(codes)[i] = make_uint2(lo, hi);
        scales[i] = (uint8_t)sb;
      }
    }
  }
}

enum Mode { kPerTensor = 0, kPerRow = 1, kGiven = 2 };

// Pass 2 (or the only pass): one lane per 16-element block, flat block index over
// rows x (cols / 16).  The grid is sized to the machine (persistent workgroups), so the
// per-tensor prologue that reduces the pass-1 partials runs once per workgroup; each
// iteration encodes two blocks whose loads are issued together.
template <typename T, int MODE>
__device__ __forceinline__ void encode_one(const T* __restrict__ x, uint32_t i, uint32_t bpr, int64_t ldx,
                                           bool dense, const FastDivU32& div_bpr, uint8_t* __restrict__ codes,
                                           uint8_t* __restrict__ scales, const float* __restrict__ row_sg,
                                           float sg, const uint4 (&w)[16 / kElemsPer16B<T>]) {
  float v[16];
#pragma unroll
  for (int c = 0; c < 16 / kElemsPer16B<T>; ++c) widen(w[c], v + c * kElemsPer16B<T>, x);
  float s = sg;
  if (MODE == kPerRow) s = row_sg[fastdiv(i, div_bpr)];
  uint32_t sb, lo, hi;
  encode_block(v, s, sb, lo, hi);
  reinterpret_cast<uint2*>(codes)[i] = make_uint2(lo, hi);
  scales[i] = (uint8_t)sb;
}

template <typename T, int MODE>
__device__ __forceinline__ const uint4* block_src(const T* __restrict__ x, uint32_t i, uint32_t bpr, int64_t ldx,
                                                  bool dense, const FastDivU32& div_bpr) {
  if (dense) return reinterpret_cast<const uint4*>(x + (int64_t)i * 16);
  const uint32_t r = fastdiv(i, div_bpr), b = i - r * bpr;
  return reinterpret_cast<const uint4*>(x + (int64_t)r * ldx + (int64_t)b * 16);
}

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void encode_kernel(const T* __restrict__ x, uint32_t rows,
                                                           uint32_t bpr, int64_t ldx, FastDivU32 div_bpr,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           float* __restrict__ global_scale,
                                                           const uint32_t* __restrict__ partial,
                                                           int npartial) {
  constexpr int NC = 16 / kElemsPer16B<T>;        // 16 B loads per block
  float sg = 0.0f;
  if (MODE == kPerTensor) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads) m = max(m, partial[i]);
    m = block_max_u32(m);
    sg = __uint_as_float(m) / kGlobalDivisor;
    if (blockIdx.x == 0 && threadIdx.x == 0) global_scale[0] = sg;
  } else if (MODE == kGiven) {
    sg = global_scale[0];
  }
  const uint32_t total = rows * bpr;
  const bool dense = ldx == (int64_t)bpr * 16;
  if (MODE == kPerTensor && dense && (gridDim.x & 7) == 0) {
    // The x-th eighth of the tensor on XCD x, in decreasing order (see amax_partial_kernel).
    const uint32_t xcd = blockIdx.x & 7;
    const uint32_t lo = (uint32_t)((uint64_t)total * xcd / 8), hi = (uint32_t)((uint64_t)total * (xcd + 1) / 8);
    const uint32_t stride = (gridDim.x >> 3) * kThreads;
    uint32_t k = (blockIdx.x >> 3) * kThreads + threadIdx.x;    // distance from the top of the eighth
    for (; k + stride < hi - lo; k += 2 * stride) {
      const uint32_t i0 = hi - 1 - k, i1 = i0 - stride;
      const uint4* p0 = block_src<T, MODE>(x, i0, bpr, ldx, true, div_bpr);
      const uint4* p1 = block_src<T, MODE>(x, i1, bpr, ldx, true, div_bpr);
      uint4 w0[NC], w1[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        w0[c] = p0[c];
        w1[c] = p1[c];
      }
      encode_one<T, MODE>(x, i0, bpr, ldx, true, div_bpr, codes, scales, global_scale, sg, w0);
      encode_one<T, MODE>(x, i1, bpr, ldx, true, div_bpr, codes, scales, global_scale, sg, w1);
    }
    if (k < hi - lo) {
      const uint32_t i0 = hi - 1 - k;
      const uint4* p0 = block_src<T, MODE>(x, i0, bpr, ldx, true, div_bpr);
      uint4 w0[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) w0[c] = p0[c];
      encode_one<T, MODE>(x, i0, bpr, ldx, true, div_bpr, codes, scales, global_scale, sg, w0);
    }
    return;
  }
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < total; i += 2 * stride) {
    const uint4* p0 = block_src<T, MODE>(x, i, bpr, ldx, dense, div_bpr);
    const uint4* p1 = block_src<T, MODE>(x, i + stride, bpr, ldx, dense, div_bpr);
    uint4 w0[NC], w1[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      w0[c] = p0[c];
      w1[c] = p1[c];
    }
    encode_one<T, MODE>(x, i, bpr, ldx, dense, div_bpr, codes, scales, global_scale, sg, w0);
    encode_one<T, MODE>(x, i + stride, bpr, ldx, dense, div_bpr, codes, scales, global_scale, sg, w1);
  }
  if (i < total) {
    const uint4* p0 = block_src<T, MODE>(x, i, bpr, ldx, dense, div_bpr);
    uint4 w0[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) w0[c] = p0[c];
    encode_one<T, MODE>(x, i, bpr, ldx, dense, div_bpr, codes, scales, global_scale, sg, w0);
  }
}

template <typename T>
int launch_typed(const T* x, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                 uint8_t* scales, float* global_scale, int mode, void* workspace,
                 hipStream_t stream) {
  const uint32_t bpr = (uint32_t)(cols / 16);
  const uint64_t total = (uint64_t)rows * bpr;
  if (mode == kPerTensor && rows == 0) {
    // max over an empty tensor is 0, so s_g = 0; write it with a one-lane launch.
    encode_kernel<T, kPerTensor><<<1, kThreads, 0, stream>>>(x, 0, bpr, ldx, make_fastdiv(bpr), codes,
                                                            scales, global_scale,
                                                            static_cast<const uint32_t*>(workspace), 0);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
  }
  if (rows == 0) return NVFP4_OK;
  DeviceInfo dev;
  const int st = device_info(stream, dev);
  if (st != NVFP4_OK) return st;
  const int cus = dev.cus;
  const uint32_t want = (uint32_t)((total + kThreads - 1) / kThreads);
  const uint32_t grid = want < (uint32_t)(8 * cus) ? want : (uint32_t)(8 * cus);
  const FastDivU32 fd = make_fastdiv(bpr);
  switch (mode) {
    case kPerTensor: {
      uint32_t* partial = static_cast<uint32_t*>(workspace);
      const int64_t chunks16 = rows * (cols / kElemsPer16B<T>);
      int64_t np64 = (chunks16 + 4 * kThreads - 1) / (4 * kThreads);
      if (ldx != cols) np64 = rows;
      int64_t cap = 4 * (int64_t)cus;
      if (cap > kMaxPartials) cap = kMaxPartials;
      const int np = (int)(np64 < cap ? np64 : cap);     // <= kMaxPartials: fits the workspace
      amax_partial_kernel<T><<<np, kThreads, 0, stream>>>(x, rows, cols, ldx, partial);
      encode_kernel<T, kPerTensor><<<grid, kThreads, 0, stream>>>(x, (uint32_t)rows, bpr, ldx, fd, codes,
                                                                  scales, global_scale, partial, np);
      break;
    }
    case kPerRow: {
      const int g = (int)(rows < 8 * cus ? rows : 8 * cus);
      constexpr int kMaxB = sizeof(T) == 2 ? 8 : 4;     // blocks per thread held in registers
      if (rows < cus && bpr <= (uint32_t)(2 * kWideThreads)) {
        if (bpr <= (uint32_t)kWideThreads)
          row_quant_kernel<T, 1, kWideThreads><<<g, kWideThreads, 0, stream>>>(x, rows, bpr, ldx, codes, scales,
                                                                                  global_scale);
        else
          row_quant_kernel<T, 2, kWideThreads><<<g, kWideThreads, 0, stream>>>(x, rows, bpr, ldx, codes, scales,
                                                                                  global_scale);
        break;
      }
      if (bpr <= (uint32_t)(kMaxB * kThreads)) {
        if (bpr <= (uint32_t)(2 * kThreads))
          row_quant_kernel<T, 2><<<g, kThreads, 0, stream>>>(x, rows, bpr, ldx, codes, scales, global_scale);
        else
          row_quant_kernel<T, kMaxB><<<g, kThreads, 0, stream>>>(x, rows, bpr, ldx, codes, scales, global_scale);
        break;
      }
      row_scale_kernel<T><<<g, kThreads, 0, stream>>>(x, rows, cols, ldx, global_scale);
      encode_kernel<T, kPerRow><<<grid, kThreads, 0, stream>>>(x, (uint32_t)rows, bpr, ldx, fd, codes,
                                                               scales, global_scale, nullptr, 0);
      break;
    }
    default:
      encode_kernel<T, kGiven><<<grid, kThreads, 0, stream>>>(x, (uint32_t)rows, bpr, ldx, fd, codes,
                                                              scales, global_scale, nullptr, 0);
      break;
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace

// The scratch array of nvfp4_quantize_no_alloc, which stands in for the caller's workspace:
// one partial max per pass-1 workgroup (4 KB).  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: launches use the address quantize_device_setup looks up once per device.
static __device__ __align__(256) uint32_t scratch[kMaxPartials];

int quantize_device_setup(void** scratch_ptr) {
  return hipGetSymbolAddress(scratch_ptr, HIP_SYMBOL(scratch)) == hipSuccess && *scratch_ptr ? NVFP4_OK
                                                                                            : NVFP4_ERR_HIP;
}

size_t quantize_scratch_bytes() { return sizeof(scratch); }

size_t quantize_workspace_bytes(int64_t, int64_t, int mode) {
  // one partial max per pass-1 workgroup, at most kMaxPartials of them
  return mode == kPerTensor ? (size_t)kMaxPartials * sizeof(uint32_t) : 0;
}

int launch_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, uint8_t* codes,
                    uint8_t* scales, float* global_scale, int mode, void* workspace, hipStream_t stream) {
  if (x_dtype == NVFP4_BF16)
    return launch_typed(static_cast<const uint16_t*>(x), rows, cols, ldx, codes, scales, global_scale, mode,
                        workspace, stream);
  return launch_typed(static_cast<const float*>(x), rows, cols, ldx, codes, scales, global_scale, mode,
                      workspace, stream);
}

}  // namespace nvfp4
