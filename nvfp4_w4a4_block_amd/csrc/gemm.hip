// Block-scaled NVFP4 x NVFP4 GEMM for gfx950: Y[M, N] = A . W^T, FP32 accumulation.
//
// What is computed (W4A4, "Why Gated DeltaNet Survives 4-Bit Quantization", "The deep
// dive"; the fused-module global-scale repair, paper abstract):
//   Y[m, n] = s_gA[m or 0] * s_gW[seg(n)] * sum_k (E2M1(a_mk) E4M3(sa_m,k/16)) (E2M1(w_nk) E4M3(sw_n,k/16))
// where seg(n) is the fused segment holding column n.
//
// Design (gfx950):
//  * Each E2M1 x E4M3 product has at most 6 significant bits and lies in [2^-10, 2688], so
//    it is exact in fp16; operands are dequantized exactly in registers and fed to the fp16
//    MFMA, whose products are exact in fp32.  Only the fp32 accumulation rounds.  The
//    global scales stay out of the operands and are applied in the epilogue, per row of A
//    and per column segment of W.
//  * Prefill kernel (M > 16): 256 x 256 output tile per 256-thread workgroup (4 wavefronts,
//    each a 128 x 128 sub-tile of 4 x 4 MFMA 32x32x16 tiles), K stages of 256.  Packed codes
//    (128 B per row per stage) and scale bytes are copied straight into LDS, double-buffered;
//    each lane reads 16 B of codes (32 elements of one row) per 64-wide K chunk and uses one
//    dword per MFMA.  The K order inside a chunk is permuted identically for A and W, which
//    leaves every dot product unchanged.  Tiles are mapped to XCDs so that each XCD's L2
//    serves a compact block of output tiles; when the last round of tiles would leave most
//    CUs idle, whole tile columns are done as 128 x 128 tiles in the same launch.
//  * Decode kernel (M <= 16): memory-bound streaming of W in one launch.  Workgroups own 32
//    rows of W and all of K, their 4 wavefronts split K, accumulate 16x16 MFMA tiles and
//    reduce them in LDS in a fixed order (deterministic) before the scales are applied.
//  * A plain kernel (one thread per output, fp32 FMA) serves shapes the fast kernels do not
//    take (K not a multiple of 128; for M > 16, K not a multiple of 256 or K >= 2^24).
//  * Epilogue modes, chosen at compile time so that each kernel keeps its registers: Y in fp32
//    or bf16; Y quantized to NVFP4 in the same launch under a given output global scale (for
//    the next linear layer); Y plus the Gated DeltaNet gates of the last two fused segments.
//  * MXFP4 operands (a lossy variant; E2M1 codes with one E8M0 scale per 32 elements): the same
//    tiles and copies, with gfx950's scaled FP4 MFMA instead of dequantization.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

struct GemmArgs {
  int32_t M, N, K;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_global;
  int32_t a_per_row;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const float* w_globals;
  void* y;
  int32_t y_bf16;
  int32_t y_vec;      // y and its row pitch allow 16-byte stores
  int64_t ldy;
  SegmentTable seg;
  int32_t q_out;      // write NVFP4 (q_codes, q_scales under q_global[0]) instead of y
  const float* q_global;
  uint8_t* q_codes;
  uint8_t* q_scales;
  int32_t gate_n0;    // GDN gates (when gate_h > 0): see store_gate
  int32_t gate_h;
  const float* gate_a_log;
  const float* gate_dt_bias;
  float* gate_g;
  float* gate_beta;
  int32_t swiglu;     // SwiGLU pairs: see store_swiglu_block (w_globals = {gate, up})
};

// Epilogue modes of the MFMA kernels.
constexpr int kEpiStore = 0;   // Y in fp32 or bf16
constexpr int kEpiNvfp4 = 1;   // Y as NVFP4 under a given global scale
constexpr int kEpiGates = 2;   // Y, and the GDN gates of the last two segments
constexpr int kEpiSwiglu = 3;  // h = silu(gate) * up of interleaved 32-column pairs

// One 16-column block of output row m (columns n .. n+15, all valid) as NVFP4: the same
// encoder as the quantizer, under the given global scale.
__device__ __forceinline__ void store_block_nvfp4(const GemmArgs& g, int m, int n, const float (&v)[16]) {
  uint32_t sb, lo, hi;
  encode_block(v, g.q_global[0], sb, lo, hi);
  *reinterpret_cast<uint2*>(g.q_codes + (int64_t)m * (g.N / 2) + n / 2) = make_uint2(lo, hi);
  g.q_scales[(int64_t)m * (g.N / 16) + n / 16] = (uint8_t)sb;
}

__device__ __forceinline__ int segment_of(int n, const SegmentTable& seg) {
  int s = 0;
  for (int i = 1; i < seg.count; ++i) s += n >= seg.bound[i];
  return s;
}

// Global scale of the weight row behind output column n: its segment's, or with SwiGLU pairs
// the gate's (columns 32p .. 32p+15) or the up projection's (32p+16 .. 32p+31).
__device__ __forceinline__ float w_global_at(const GemmArgs& g, int n) {
  return g.swiglu ? g.w_globals[(n >> 4) & 1] : g.w_globals[segment_of(n, g.seg)];
}

__device__ __forceinline__ void store_out(const GemmArgs& g, int m, int n, float v) {
  if (g.y_bf16)
    static_cast<uint16_t*>(g.y)[(int64_t)m * g.ldy + n] = f32_to_bf16_rne(v);
  else
    static_cast<float*>(g.y)[(int64_t)m * g.ldy + n] = v;
}

// The Gated DeltaNet gates of one fp32 output value y at row m, column n >= gate_n0 (the two
// gate projections end the fused GDN input projection; "Why Gated DeltaNet Survives 4-Bit
// Quantization", "The deep dive": the write strength goes through a sigmoid, the decay is
// parameterized in log space through softplus and exponential).  Column gate_n0 + j is head j
// of the write strength, beta = 1 / (1 + e^-y); column gate_n0 + gate_h + j is head j of the
// decay, g = -e^A_log[j] * softplus(y + dt_bias[j]) with softplus(z) = max(z, 0) + ln(1 + e^-|z|),
// which overflows nowhere.
__device__ __forceinline__ float gate_write_strength(float y) { return 1.0f / (1.0f + expf(-y)); }

// e_alog = e^A_log[j] of the head, dt = dt_bias[j].
__device__ __forceinline__ float gate_log_decay(float y, float e_alog, float dt) {
  const float z = y + dt;
  const float sp = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
  return -e_alog * sp;
}

__device__ __forceinline__ void store_gate(const GemmArgs& g, int m, int n, float y) {
  const int c = n - g.gate_n0;
  if (c < g.gate_h) {
    g.gate_beta[(int64_t)m * g.gate_h + c] = gate_write_strength(y);
  } else {
    const int j = c - g.gate_h;
    g.gate_g[(int64_t)m * g.gate_h + j] = gate_log_decay(y, expf(g.gate_a_log[j]), g.gate_dt_bias[j]);
  }
}

// SiLU of an fp32 GEMM output, y * sigmoid(y) = y / (1 + e^-y) (the gated MLP's activation),
// with the hardware base-2 exponential and reciprocal, each within one ulp: the result's
// relative error is at most about (|y| + 3) 2^-23, the |y| part from rounding the exponential's
// argument -y log2(e) to fp32.  For y below about -88 the exponential overflows and the result
// is -0, where the exact value is under 3e-37.
__device__ __forceinline__ float silu(float y) {
  const float e = __builtin_amdgcn_exp2f(-y * 1.44269504088896341f);   // log2(e)
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// SwiGLU of one interleaved column pair of output row m: fused columns n .. n+15 (n a multiple
// of 32) are gate outputs and n+16 .. n+31 the up outputs of the same 16 hidden units
// n/2 .. n/2+15, so h = silu(gate) * up is one 16-element block of the hidden row (width N/2).
// gv and uv hold the 16 fp32 outputs (global scales applied) each, 16-byte aligned.  h is stored
// as fp32 or bf16 when y is given (row pitch ldy) and as one NVFP4 block under q_global[0]
// when q_out (codes [M, N/4], scale bytes [M, N/32]).
__device__ __forceinline__ void store_swiglu_block(const GemmArgs& g, int m, int n, const float* gv,
                                                   const float* uv) {
  float h[16];
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 a = *reinterpret_cast<const float4*>(gv + e);
    const float4 b = *reinterpret_cast<const float4*>(uv + e);
    h[e] = silu(a.x) * b.x;
    h[e + 1] = silu(a.y) * b.y;
    h[e + 2] = silu(a.z) * b.z;
    h[e + 3] = silu(a.w) * b.w;
  }
  const int j = n >> 1;                       // first hidden column of the block
  if (g.y) {
    if (g.y_bf16) {
      uint16_t* y = static_cast<uint16_t*>(g.y) + (int64_t)m * g.ldy + j;
      if (g.y_vec) {
        uint4* y4 = reinterpret_cast<uint4*>(y);
        y4[0] = make_uint4(bf16_pair(h[0], h[1]), bf16_pair(h[2], h[3]), bf16_pair(h[4], h[5]), bf16_pair(h[6], h[7]));
        y4[1] = make_uint4(bf16_pair(h[8], h[9]), bf16_pair(h[10], h[11]), bf16_pair(h[12], h[13]),
                           bf16_pair(h[14], h[15]));
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) y[e] = f32_to_bf16_rne(h[e]);
      }
    } else {
      float* y = static_cast<float*>(g.y) + (int64_t)m * g.ldy + j;
      if (g.y_vec) {
#pragma unroll
        for (int e = 0; e < 16; e += 4) *reinterpret_cast<float4*>(y + e) = make_float4(h[e], h[e + 1], h[e + 2], h[e + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) y[e] = h[e];
      }
    }
  }
  if (g.q_out) {
    uint32_t sb, lo, hi;
    encode_block(h, g.q_global[0], sb, lo, hi);
    const int64_t width = g.N >> 1;
    *reinterpret_cast<uint2*>(g.q_codes + (int64_t)m * (width / 2) + j / 2) = make_uint2(lo, hi);
    g.q_scales[(int64_t)m * (width / 16) + j / 16] = (uint8_t)sb;
  }
}

// Byte k of a dword as an fp16 scale pair (E4M3 * 2^-8 in both halves).
__device__ __forceinline__ half2_t pair_of_byte(uint32_t dw, int k) {
  return scale_pair_f16((dw >> (8 * k)) & 0xFFu);
}

// ------------------------------------------------------------------ prefill kernel

constexpr int BK = 256;
constexpr int kRowBytes = BK / 2;           // 128 B of codes per row per K step
constexpr int kScaleRow = BK / 16;          // 16 scale bytes per row per K step
constexpr int kChunks = BK / 64;            // 64-wide chunks per K step
constexpr int kStages = 2;
constexpr int kPrefillThreads = 256;

// Stage layout for a T x T output tile: codes of A (T rows x 128 B), codes of W, scale bytes
// of A (T rows x 16 B), scale bytes of W.
template <int T> struct TileCfg {
  static constexpr int kCodeTile = T * kRowBytes;
  static constexpr int kScaleTile = T * kScaleRow;
  static constexpr int kStageBytes = 2 * kCodeTile + 2 * kScaleTile;
  static constexpr int F = T / 64;           // MFMA 32x32 tiles per wavefront per dimension
};
// Behind the stage buffers: the tile's row and column global scales (256 floats each).
constexpr int kScaleTableOffset = kStages * TileCfg<256>::kStageBytes;
constexpr int kPrefillLds = kScaleTableOffset + 2 * 256 * 4;

typedef __attribute__((address_space(3))) void lds_void_t;

// Rows of codes are unpadded; the eight 16 B slots of a row are XOR-swizzled with
// slot_swizzle(row) so that fragment reads (16 consecutive rows, one slot each) hit distinct
// LDS bank groups whether the LDS serves 128 B or 256 B per cycle.
__device__ __forceinline__ int slot_swizzle(int row) { return (row ^ (row >> 3)) & 7; }

// Copy 16 B per lane from global memory straight into LDS: lane l reads base + off (off a
// per-lane byte offset, base the same for the whole wavefront) and its bytes land at
// lds_dst + 16 l (1 KB of consecutive LDS per wavefront).  Issued from inline assembly on
// purpose: the compiler then does not treat the copy as an LDS store that every later LDS
// read must wait for (it cannot tell the two stage buffers apart).  The copy writes no
// registers; the K loop orders it explicitly: a stage's copies are waited for (vmcnt(0)) and
// published with a barrier before any wavefront reads that stage, and they are issued only
// after a barrier that follows every read of the buffer they overwrite.  lds_dst must be the
// same for every lane.  M0 cannot be named as clobbered (the compiler reserves it); nothing
// else in this file's kernels uses M0, which a CPU test checks on the generated assembly.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* base, uint32_t off, const uint8_t* lds_dst) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds_dst);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "s"(dst) : "memory");
}

// The same with 4 B per lane (lane l lands at lds_dst + 4 l: 256 B per wavefront).
__device__ __forceinline__ void copy4_to_lds(const uint8_t* base, uint32_t off, const uint8_t* lds_dst) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds_dst);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" : : "v"(off), "s"(base), "s"(dst) : "memory");
}

// Enqueue the copy of K step kt of both operands straight into LDS (no registers): each
// wavefront-wide load writes 1 KB of consecutive LDS (8 rows of codes, or 64 rows of scales).
// Rows past the end of A or W are clamped to the last row.  Addresses are a per-tile base in
// scalar registers plus a 32-bit per-lane offset, row * row pitch + segment, with row < 256 and
// the pitch < 2^23 (K < 2^24), so 24-bit multiplies serve.  MX: the operands are MXFP4, whose
// 8 E8M0 bytes per row per K step land in the scale area with a row pitch of 8 B (4 B per lane).
template <int T, bool MX = false>
__device__ __forceinline__ void load_stage_lds(const GemmArgs& g, int m0, int n0, int kt, uint8_t* stage) {
  using C = TileCfg<T>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const uint32_t kb = (uint32_t)g.K / 2, ks = (uint32_t)g.K / 16;
  const int ra = g.M - 1 - m0, rw = g.N - 1 - n0;          // last valid tile row of A, W
  const uint8_t* ac = g.a_codes + (size_t)m0 * kb + (size_t)kt * kRowBytes;
  const uint8_t* wc = g.w_codes + (size_t)n0 * kb + (size_t)kt * kRowBytes;
  const uint8_t* as = g.a_scales + (size_t)m0 * ks + (size_t)kt * kScaleRow;
  const uint8_t* ws = g.w_scales + (size_t)n0 * ks + (size_t)kt * kScaleRow;
#pragma unroll
  for (int j = 0; j < T / 32; ++j) {
    const int chunk = j * 4 + wave;                  // 1 KB chunk = 8 rows
    const int row = chunk * 8 + (lane >> 3);
    const uint32_t seg = (uint32_t)(((lane & 7) ^ slot_swizzle(row)) * 16);  // logical 16 B segment in slot lane&7
    copy16_to_lds(ac, __umul24(min(row, ra), kb) + seg, stage + chunk * 1024);
    copy16_to_lds(wc, __umul24(min(row, rw), kb) + seg, stage + C::kCodeTile + chunk * 1024);
  }
  if constexpr (MX) {
    const uint32_t kx = (uint32_t)g.K / 32;
    const uint8_t* ax = g.a_scales + (size_t)m0 * kx + (size_t)kt * 8;
    const uint8_t* wx = g.w_scales + (size_t)n0 * kx + (size_t)kt * 8;
#pragma unroll
    for (int j = 0; j < T / 128; ++j) {
      const int chunk = j * 4 + wave;                // 256 B chunk = 32 rows x 8 B
      const int row = chunk * 32 + (lane >> 1);
      const uint32_t half = (uint32_t)(lane & 1) * 4;
      copy4_to_lds(ax, __umul24(min(row, ra), kx) + half, stage + 2 * C::kCodeTile + chunk * 256);
      copy4_to_lds(wx, __umul24(min(row, rw), kx) + half, stage + 2 * C::kCodeTile + C::kScaleTile + chunk * 256);
    }
  } else {
#pragma unroll
    for (int j = 0; j < T / 256; ++j) {
      const int chunk = j * 4 + wave;                // 1 KB chunk = 64 rows x 16 B
      const int row = chunk * 64 + lane;
      copy16_to_lds(as, __umul24(min(row, ra), ks), stage + 2 * C::kCodeTile + chunk * 1024);
      copy16_to_lds(ws, __umul24(min(row, rw), ks), stage + 2 * C::kCodeTile + C::kScaleTile + chunk * 1024);
    }
    if (T / 256 == 0) {   // 128-row tiles: 128 rows x 16 B = 2 KB per operand, half the waves each
      const int row = (wave & 1) * 64 + lane;
      if (wave < 2)
        copy16_to_lds(as, __umul24(min(row, ra), ks), stage + 2 * C::kCodeTile + (wave & 1) * 1024);
      else
        copy16_to_lds(ws, __umul24(min(row, rw), ks), stage + 2 * C::kCodeTile + C::kScaleTile + (wave & 1) * 1024);
    }
  }
}

// Tile index -> (tile_m, tile_n).  Workgroups are dispatched round-robin over the 8 XCDs;
// workgroup i is given logical tile start(i % 8) + i / 8, so each XCD owns a contiguous
// range of logical tiles, ordered in groups of 8 tile rows (column-major inside a group)
// so that concurrently resident tiles share rows of A and W in that XCD's L2.
__device__ __forceinline__ void tile_coords(int i, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int x = i & 7, j = i >> 3;
  const int per = T >> 3, rem = T & 7;
  const int t = x * per + min(x, rem) + j;
  const int G = 8;
  const int group = t / (G * tiles_n);
  const int first = group * G;
  const int gsize = min(tiles_m - first, G);
  const int in = t - group * G * tiles_n;
  tm = first + in % gsize;
  tn = in / gsize;
}

// The two scale bytes of a lane's 32 elements of a 64-wide chunk (bytes 2h and 2h+1 of the
// chunk's scale dword, picked by sel) as fp16 E4M3 * 2^-8 in the low and high half of one
// register: the same bits scale_pair_f16 gives each byte.
__device__ __forceinline__ uint32_t scale_halves(uint32_t dw, uint32_t sel) {
  return __builtin_amdgcn_perm(0u, dw, sel) << 7;
}

// Selector for scale_halves: bytes 2h and 2h+1 to bytes 0 and 2, zeros elsewhere.
__device__ __forceinline__ uint32_t scale_halves_sel(int h) { return h ? 0x0c030c02u : 0x0c010c00u; }

// Dequantize the fragments of one 16-deep K step (step s of a 64-wide chunk) for the F A
// and F W row groups of this wavefront: dword s of each lane's 16 B of codes, scaled by
// the scale of block (2h + s/2) of the chunk (low half of pa/pb for s < 2, else high half).
template <int F>
__device__ __forceinline__ void dequant_step(const uint4 (&qa)[F], const uint4 (&qb)[F], const uint32_t (&pa)[F],
                                             const uint32_t (&pb)[F], int s, half8_t (&fa)[F],
                                             half8_t (&fb)[F]) {
#pragma unroll
  for (int i = 0; i < F; ++i) {
    const uint32_t wa = s == 0 ? qa[i].x : s == 1 ? qa[i].y : s == 2 ? qa[i].z : qa[i].w;
    const uint32_t wb = s == 0 ? qb[i].x : s == 1 ? qb[i].y : s == 2 ? qb[i].z : qb[i].w;
    const half2_t ha = __builtin_bit_cast(half2_t, pa[i]), hb = __builtin_bit_cast(half2_t, pb[i]);
    fa[i] = dequant8_f16(wa, s < 2 ? half2_t{ha[0], ha[0]} : half2_t{ha[1], ha[1]});
    fb[i] = dequant8_f16(wb, s < 2 ? half2_t{hb[0], hb[0]} : half2_t{hb[1], hb[1]});
  }
}

// Registers one wave carries through the K loop of a T x T tile.
template <int T>
struct PrefillRegs {
  static constexpr int F = T / 64;
  f32x16_t acc[F][F];
  uint4 sa[F], sb[F], qa[F], qb[F];   // scale bytes of the stage, codes of the current chunk
  uint32_t pa[F], pb[F];              // scales of the current chunk (scale_halves)
  uint32_t sel;                       // scale_halves selector of this lane
  half8_t fa[F], fb[F];               // fragments of the current step
  int swa[F], swb[F];                 // slot swizzles of the lane's rows
};

// One 256-deep stage kt of a tile, as 16 steps of 16-deep MFMAs.  Step 12 waits for stage
// kt+1's copies and publishes them with the stage's only barrier; right after it the copies
// of stage kt+2 are issued into stage kt's buffer when LOAD (no wave reads that buffer after
// step 10).  Stage kt+1's scales and first codes are read at steps 13 and 14 and its first
// fragments dequantized during step 15, so every stage starts straight with MFMAs.  In the
// last stage that look-ahead reads a stale buffer and its results are never used; keeping
// it unconditional keeps the loop free of branches.
template <int T, bool LOAD>
__device__ __forceinline__ void prefill_stage(const GemmArgs& g, uint8_t* lds, int m0, int n0, int kt,
                                              PrefillRegs<T>& R) {
  using C = TileCfg<T>;
  constexpr int F = C::F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * (T / 2), wn = (wave & 1) * (T / 2);
  const int r = lane & 31, h = lane >> 5;
  uint8_t* buf = lds + (kt & 1) * C::kStageBytes;
  const uint8_t* nbuf = lds + ((kt + 1) & 1) * C::kStageBytes;
#pragma unroll
  for (int step = 0; step < 4 * kChunks; ++step) {
    __builtin_amdgcn_sched_barrier(0);
    const int c = step >> 2;
    if (step == 12) {
      __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): stage kt+1 copied by this wave
      __syncthreads();                           // ... and by every wave
      if (LOAD) load_stage_lds<T>(g, m0, n0, kt + 2, buf);
    }
    if (step == 13) {
      const uint8_t* sa_t = nbuf + 2 * C::kCodeTile + (wm + r) * kScaleRow;
      const uint8_t* sb_t = nbuf + 2 * C::kCodeTile + C::kScaleTile + (wn + r) * kScaleRow;
#pragma unroll
      for (int i = 0; i < F; ++i) {
        R.sa[i] = *reinterpret_cast<const uint4*>(sa_t + 32 * i * kScaleRow);
        R.sb[i] = *reinterpret_cast<const uint4*>(sb_t + 32 * i * kScaleRow);
      }
    }
    if ((step & 3) == 3) {
      // scale pairs of the next chunk (this stage's chunk c+1, or the next stage's chunk 0)
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const uint32_t da = c == 0 ? R.sa[i].y : c == 1 ? R.sa[i].z : c == 2 ? R.sa[i].w : R.sa[i].x;
        const uint32_t db = c == 0 ? R.sb[i].y : c == 1 ? R.sb[i].z : c == 2 ? R.sb[i].w : R.sb[i].x;
        R.pa[i] = scale_halves(da, R.sel);
        R.pb[i] = scale_halves(db, R.sel);
      }
    }
    half8_t na[F], nb[F];
    dequant_step<F>(R.qa, R.qb, R.pa, R.pb, (step + 1) & 3, na, nb);
    if ((step & 3) == 2) {
      // chunk c's codes are dequantized to the end now: read the next chunk's codes
      const uint8_t* src = c + 1 < kChunks ? buf : nbuf;
      const int slot = c + 1 < kChunks ? 2 * (c + 1) + h : h;
      const uint8_t* ca = src + (wm + r) * kRowBytes;
      const uint8_t* cb = src + C::kCodeTile + (wn + r) * kRowBytes;
#pragma unroll
      for (int i = 0; i < F; ++i) {
        R.qa[i] = *reinterpret_cast<const uint4*>(ca + 32 * i * kRowBytes + ((slot ^ R.swa[i]) << 4));
        R.qb[i] = *reinterpret_cast<const uint4*>(cb + 32 * i * kRowBytes + ((slot ^ R.swb[i]) << 4));
      }
    }
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j)
        R.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(R.fa[i], R.fb[j], R.acc[i][j], 0, 0, 0);
    // Interleave: one MFMA, then the next step's dequantization spread between them.
#pragma unroll
    for (int k = 0; k < F * F; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 16 / F, 0);
    }
#pragma unroll
    for (int i = 0; i < F; ++i) {
      R.fa[i] = na[i];
      R.fb[i] = nb[i];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------ MXFP4 operands

// Registers one wave carries through the K loop of a T x T tile whose operands are MXFP4
// (E2M1 codes with one E8M0 scale per 32 elements).
template <int T>
struct MxRegs {
  static constexpr int F = T / 64;
  f32x16_t acc[F][F];
  uint4 qa[F], qb[F];            // codes of the current 64-wide chunk: the lane's 32-element block
  uint32_t sa[2][F], sb[2][F];   // the stage's 8 E8M0 bytes of each lane row: byte 2 (c & 1) + h of
                                 // dword c >> 1 is block 2c + h
  int swa[F], swb[F];
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8_t fp4_operand(const uint4& q) {
  return i32x8_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
}

// The F x F scaled MFMAs of one 64-wide chunk: lane (r, h) supplies the 32 E2M1 codes of block
// 2c + h of its A row and W row and their E8M0 bytes, byte OPSEL + h of the scale dwords (the
// dwords are shifted right by sh = 8h here, at their use, so that OPSEL is the same for every
// lane).  The hardware scales each product by 2^(sa - 127) * 2^(sb - 127) and accumulates in fp32.
template <int F, int OPSEL>
__device__ __forceinline__ void mx_chunk_mma(f32x16_t (&acc)[F][F], const uint4 (&qa)[F], const uint4 (&qb)[F],
                                             const uint32_t (&sa)[F], const uint32_t (&sb)[F], uint32_t sh) {
  int xa[F], xb[F];
#pragma unroll
  for (int i = 0; i < F; ++i) {
    xa[i] = (int)(sa[i] >> sh);
    xb[i] = (int)(sb[i] >> sh);
  }
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(qa[i]), fp4_operand(qb[j]), acc[i][j],
                                                                  4, 4, OPSEL, xa[i], OPSEL, xb[j]);
}

// One 256-deep stage kt of an MXFP4 tile, as 4 chunks of 64-deep scaled MFMAs.  While a chunk's
// MFMAs run, the next chunk's codes are read from LDS; before the last chunk the stage kt+1
// copies are waited for and published with the stage's only barrier, the copies of stage kt+2
// are issued into stage kt's buffer when LOAD (every read of it is done), and the next stage's
// first codes and scale bytes are read.  In the last stage that look-ahead reads a stale
// buffer whose values are never used.
template <int T, bool LOAD>
__device__ __forceinline__ void mx_stage(const GemmArgs& g, uint8_t* lds, int m0, int n0, int kt, MxRegs<T>& R) {
  using C = TileCfg<T>;
  constexpr int F = C::F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * (T / 2), wn = (wave & 1) * (T / 2);
  const int r = lane & 31, h = lane >> 5;
  uint8_t* buf = lds + (kt & 1) * C::kStageBytes;
  const uint8_t* nbuf = lds + ((kt + 1) & 1) * C::kStageBytes;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    const bool last = c + 1 == kChunks;
    if (last) {
      __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): stage kt+1 copied by this wave
      __syncthreads();                           // ... and by every wave
      if (LOAD) load_stage_lds<T, true>(g, m0, n0, kt + 2, buf);
    }
    const uint8_t* src = last ? nbuf : buf;
    const int slot = last ? h : 2 * (c + 1) + h;
    const uint8_t* ca = src + (wm + r) * kRowBytes;
    const uint8_t* cb = src + C::kCodeTile + (wn + r) * kRowBytes;
    uint4 na[F], nb[F];
#pragma unroll
    for (int i = 0; i < F; ++i) {
      na[i] = *reinterpret_cast<const uint4*>(ca + 32 * i * kRowBytes + ((slot ^ R.swa[i]) << 4));
      nb[i] = *reinterpret_cast<const uint4*>(cb + 32 * i * kRowBytes + ((slot ^ R.swb[i]) << 4));
    }
    uint32_t nsa[2][F], nsb[2][F];
    if (last) {
      const uint8_t* sa_t = nbuf + 2 * C::kCodeTile + (wm + r) * 8;
      const uint8_t* sb_t = nbuf + 2 * C::kCodeTile + C::kScaleTile + (wn + r) * 8;
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const uint2 xa = *reinterpret_cast<const uint2*>(sa_t + 32 * i * 8);
        const uint2 xb = *reinterpret_cast<const uint2*>(sb_t + 32 * i * 8);
        nsa[0][i] = xa.x;
        nsa[1][i] = xa.y;
        nsb[0][i] = xb.x;
        nsb[1][i] = xb.y;
      }
    }
    const uint32_t sh = 8u * (uint32_t)h;
    if ((c & 1) == 0)
      mx_chunk_mma<F, 0>(R.acc, R.qa, R.qb, R.sa[c >> 1], R.sb[c >> 1], sh);
    else
      mx_chunk_mma<F, 2>(R.acc, R.qa, R.qb, R.sa[c >> 1], R.sb[c >> 1], sh);
    // Issue order: the look-ahead LDS reads first, one between consecutive MFMAs, so that they
    // complete long before the next chunk needs them.
    constexpr int kMma = F * F;
    const int reads = last ? 4 * F : 2 * F;
#pragma unroll
    for (int k = 0; k < 4 * F; ++k) {
      if (k < reads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (k < kMma) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if (kMma > 4 * F) __builtin_amdgcn_sched_group_barrier(0x008, kMma - 4 * F, 0);
#pragma unroll
    for (int i = 0; i < F; ++i) {
      R.qa[i] = na[i];
      R.qb[i] = nb[i];
    }
    if (last) {
#pragma unroll
      for (int i = 0; i < F; ++i) {
        R.sa[0][i] = nsa[0][i];
        R.sa[1][i] = nsa[1][i];
        R.sb[0][i] = nsb[0][i];
        R.sb[1][i] = nsb[1][i];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One T x T output tile (T = 256 or 128) on 4 waves in a 2 x 2 grid, each wave T/2 x T/2 as
// (T/64) x (T/64) MFMA 32x32x16 f16 tiles, over the whole K range in 256-deep stages
// double-buffered in LDS.
template <int T, int EPI, bool MX = false>
__device__ __forceinline__ void prefill_tile(const GemmArgs& g, uint8_t* lds, int m0, int n0) {
  using C = TileCfg<T>;
  constexpr int F = C::F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = (wave >> 1) * (T / 2), wn = (wave & 1) * (T / 2);
  const int r = lane & 31, h = lane >> 5;
  std::conditional_t<MX, MxRegs<T>, PrefillRegs<T>> R;
  if constexpr (!MX) R.sel = scale_halves_sel(h);
#pragma unroll
  for (int i = 0; i < F; ++i) {
    R.swa[i] = slot_swizzle(wm + 32 * i + r);
    R.swb[i] = slot_swizzle(wn + 32 * i + r);
  }
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j) R.acc[i][j] = f32x16_t{};

  // Prologue: stages 0 and 1 in flight, the scale tables filled, stage 0 published, its
  // first step's fragments made.
  const int nk = g.K / BK;
  load_stage_lds<T, MX>(g, m0, n0, 0, lds);
  if (nk > 1) load_stage_lds<T, MX>(g, m0, n0, 1, lds + C::kStageBytes);
  {
    float* row_scale = reinterpret_cast<float*>(lds + kScaleTableOffset);
    for (int t = threadIdx.x; t < 2 * T; t += kPrefillThreads) {
      const int n = min(n0 + t - T, g.N - 1);
      row_scale[t] = t < T ? g.a_global[g.a_per_row ? min(m0 + t, g.M - 1) : 0]
                           : g.w_globals[EPI == kEpiSwiglu ? (n >> 4) & 1 : segment_of(n, g.seg)];
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
  __syncthreads();
  if constexpr (MX) {
    const uint8_t* ca = lds + (wm + r) * kRowBytes;
    const uint8_t* cb = lds + C::kCodeTile + (wn + r) * kRowBytes;
    const uint8_t* sa_t = lds + 2 * C::kCodeTile + (wm + r) * 8;
    const uint8_t* sb_t = lds + 2 * C::kCodeTile + C::kScaleTile + (wn + r) * 8;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      R.qa[i] = *reinterpret_cast<const uint4*>(ca + 32 * i * kRowBytes + ((h ^ R.swa[i]) << 4));
      R.qb[i] = *reinterpret_cast<const uint4*>(cb + 32 * i * kRowBytes + ((h ^ R.swb[i]) << 4));
      const uint2 xa = *reinterpret_cast<const uint2*>(sa_t + 32 * i * 8);
      const uint2 xb = *reinterpret_cast<const uint2*>(sb_t + 32 * i * 8);
      R.sa[0][i] = xa.x;
      R.sa[1][i] = xa.y;
      R.sb[0][i] = xb.x;
      R.sb[1][i] = xb.y;
    }
  } else {
    const uint8_t* ca = lds + (wm + r) * kRowBytes;
    const uint8_t* cb = lds + C::kCodeTile + (wn + r) * kRowBytes;
    const uint8_t* sa_t = lds + 2 * C::kCodeTile + (wm + r) * kScaleRow;
    const uint8_t* sb_t = lds + 2 * C::kCodeTile + C::kScaleTile + (wn + r) * kScaleRow;
#pragma unroll
    for (int i = 0; i < F; ++i) {
      R.sa[i] = *reinterpret_cast<const uint4*>(sa_t + 32 * i * kScaleRow);
      R.sb[i] = *reinterpret_cast<const uint4*>(sb_t + 32 * i * kScaleRow);
      R.qa[i] = *reinterpret_cast<const uint4*>(ca + 32 * i * kRowBytes + ((h ^ R.swa[i]) << 4));
      R.qb[i] = *reinterpret_cast<const uint4*>(cb + 32 * i * kRowBytes + ((h ^ R.swb[i]) << 4));
    }
#pragma unroll
    for (int i = 0; i < F; ++i) {
      R.pa[i] = scale_halves(R.sa[i].x, R.sel);
      R.pb[i] = scale_halves(R.sb[i].x, R.sel);
    }
    dequant_step<F>(R.qa, R.qb, R.pa, R.pb, 0, R.fa, R.fb);
  }
  int kt = 0;
  if constexpr (MX) {
    for (; kt + 2 < nk; ++kt) mx_stage<T, true>(g, lds, m0, n0, kt, R);
    for (; kt < nk; ++kt) mx_stage<T, false>(g, lds, m0, n0, kt, R);
  } else {
    for (; kt + 2 < nk; ++kt) prefill_stage<T, true>(g, lds, m0, n0, kt, R);
    for (; kt < nk; ++kt) prefill_stage<T, false>(g, lds, m0, n0, kt, R);
  }
  auto& acc = R.acc;

  // Epilogue: y = (acc * s_gA[m]) * s_gW[seg(n)], with the scales from the tables.
  const float* row_scale = reinterpret_cast<const float*>(lds + kScaleTableOffset);
  const float* col_scale = row_scale + T;
  float sw[F];
#pragma unroll
  for (int j = 0; j < F; ++j) sw[j] = col_scale[wn + 32 * j + r];
  if constexpr (EPI == kEpiNvfp4 || EPI == kEpiGates || EPI == kEpiSwiglu) {
    // The scaled fp32 results go through LDS in passes of 128 tile rows (row pitch T + 8
    // floats, so the two row groups one write touches use disjoint banks).  NVFP4 output: each
    // thread then encodes whole 16-column blocks of a row.  SwiGLU: each thread takes whole
    // 32-column gate/up pairs of a row.  Gates: the tile's gate columns are read back, one
    // value per thread and step; tiles without gate columns skip this.
    constexpr int kQPitch = T + 8;
    constexpr int kQPasses = T / 128;
    constexpr int kBlocksPerRow = T / 16;
    float* out = reinterpret_cast<float*>(lds);
    int c0 = 0, c1 = 0;
    if constexpr (EPI == kEpiGates) {
      c0 = max(n0, g.gate_n0);
      c1 = min(n0 + T, g.N);
    }
    if (EPI != kEpiGates || c0 < c1) {
      __syncthreads();
#pragma unroll
      for (int p = 0; p < kQPasses; ++p) {
        if (wm == 128 * p || kQPasses == 1) {
#pragma unroll
          for (int i = 0; i < F; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
              const int tr = wm + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);   // row in the tile
              const float sam = row_scale[tr];
#pragma unroll
              for (int j = 0; j < F; ++j)
                out[(tr - 128 * p) * kQPitch + wn + 32 * j + r] = (acc[i][j][q] * sam) * sw[j];
            }
        }
        __syncthreads();
        if constexpr (EPI == kEpiNvfp4) {
          for (int b = threadIdx.x; b < 128 * kBlocksPerRow; b += kPrefillThreads) {
            const int lr = b / kBlocksPerRow, cb = b % kBlocksPerRow;
            const int m = m0 + 128 * p + lr, n = n0 + 16 * cb;
            if (m < g.M && n < g.N) {
              float v[16];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float4 f = *reinterpret_cast<const float4*>(out + lr * kQPitch + 16 * cb + 4 * e);
                v[4 * e] = f.x;
                v[4 * e + 1] = f.y;
                v[4 * e + 2] = f.z;
                v[4 * e + 3] = f.w;
              }
              store_block_nvfp4(g, m, n, v);
            }
          }
        } else if constexpr (EPI == kEpiSwiglu) {
          constexpr int kPairsPerRow = T / 32;
          for (int b = threadIdx.x; b < 128 * kPairsPerRow; b += kPrefillThreads) {
            const int lr = b / kPairsPerRow, pj = b % kPairsPerRow;
            const int m = m0 + 128 * p + lr, n = n0 + 32 * pj;
            const float* v = out + lr * kQPitch + 32 * pj;
            if (m < g.M && n < g.N) store_swiglu_block(g, m, n, v, v + 16);
          }
        } else {
          // One gate segment at a time, so that a wavefront evaluates one function; a lane
          // keeps its column's head parameters in registers across the rows.
          for (int sg = 0; sg < 2; ++sg) {
            const int sb = g.gate_n0 + sg * g.gate_h;
            const int hi = min(c1, sb + g.gate_h);
            for (int n = max(c0, sb) + lane; n < hi; n += 64) {
              const int j = n - sb;
              const float e_alog = sg ? expf(g.gate_a_log[j]) : 0.0f;
              const float dt = sg ? g.gate_dt_bias[j] : 0.0f;
              float* dst = (sg ? g.gate_g : g.gate_beta) + j;
              for (int lr = wave; lr < 128; lr += kPrefillThreads / 64) {
                const int m = m0 + 128 * p + lr;
                if (m >= g.M) break;
                const float y = out[lr * kQPitch + (n - n0)];
                dst[(int64_t)m * g.gate_h] = sg ? gate_log_decay(y, e_alog, dt) : gate_write_strength(y);
              }
            }
          }
        }
        if (p + 1 < kQPasses) __syncthreads();
      }
    }
    if constexpr (EPI == kEpiNvfp4 || EPI == kEpiSwiglu) return;
  }
  if (!g.y_bf16) {
    // fp32: each store instruction covers 128 contiguous bytes of two rows; store directly.
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int lr = wm + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
        if (m0 + lr >= g.M) continue;
        const float sam = row_scale[lr];
#pragma unroll
        for (int j = 0; j < F; ++j) {
          const int n = n0 + wn + 32 * j + r;
          if (n < g.N) store_out(g, m0 + lr, n, (acc[i][j][q] * sam) * sw[j]);
        }
      }
    return;
  }
  // bf16: the rounded results go through LDS (free once every wave has left the K loop) so
  // that rows leave as whole 16-byte segments.  A lane holds rows 2u and 2u+1 of a column in
  // consecutive accumulator registers; they are packed into one dword of row pair u, column
  // n.  Pitch T + 16 dwords per row pair: the two row pairs one write touches fall in
  // disjoint LDS banks.
  constexpr int kPitch = T + 16;
  constexpr int kVecPerPair = T / 8;
  constexpr int kPairsPerIter = kPrefillThreads / kVecPerPair;
  uint32_t* out = reinterpret_cast<uint32_t*>(lds);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int lr = wm + 32 * i + 8 * g4 + 4 * h;          // rows lr .. lr+3 of this lane
      const float4 sam = *reinterpret_cast<const float4*>(row_scale + lr);
#pragma unroll
      for (int j = 0; j < F; ++j) {
        const int col = wn + 32 * j + r;
        const f32x16_t& c = acc[i][j];
        out[(lr >> 1) * kPitch + col] =
            bf16_pair((c[4 * g4] * sam.x) * sw[j], (c[4 * g4 + 1] * sam.y) * sw[j]);
        out[((lr >> 1) + 1) * kPitch + col] =
            bf16_pair((c[4 * g4 + 2] * sam.z) * sw[j], (c[4 * g4 + 3] * sam.w) * sw[j]);
      }
    }
  __syncthreads();
  const int c8 = ((int)threadIdx.x % kVecPerPair) * 8;
  const int n = n0 + c8;
  const bool vec = g.y_vec && n + 8 <= g.N;
  uint16_t* y = static_cast<uint16_t*>(g.y);
#pragma unroll 4
  for (int it = 0; it < T / 2 / kPairsPerIter; ++it) {
    const int u = it * kPairsPerIter + (int)threadIdx.x / kVecPerPair;
    const int m = m0 + 2 * u;
    if (m >= g.M) continue;
    const uint4 p0 = *reinterpret_cast<const uint4*>(out + u * kPitch + c8);
    const uint4 p1 = *reinterpret_cast<const uint4*>(out + u * kPitch + c8 + 4);
    // low halves -> row 2u, high halves -> row 2u+1
    uint4 r0, r1;
    r0.x = __builtin_amdgcn_perm(p0.y, p0.x, 0x05040100u);
    r0.y = __builtin_amdgcn_perm(p0.w, p0.z, 0x05040100u);
    r0.z = __builtin_amdgcn_perm(p1.y, p1.x, 0x05040100u);
    r0.w = __builtin_amdgcn_perm(p1.w, p1.z, 0x05040100u);
    r1.x = __builtin_amdgcn_perm(p0.y, p0.x, 0x07060302u);
    r1.y = __builtin_amdgcn_perm(p0.w, p0.z, 0x07060302u);
    r1.z = __builtin_amdgcn_perm(p1.y, p1.x, 0x07060302u);
    r1.w = __builtin_amdgcn_perm(p1.w, p1.z, 0x07060302u);
    const bool second = m + 1 < g.M;
    if (vec) {
      *reinterpret_cast<uint4*>(y + (int64_t)m * g.ldy + n) = r0;
      if (second) *reinterpret_cast<uint4*>(y + (int64_t)(m + 1) * g.ldy + n) = r1;
    } else {
      const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w}, w1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (n + k >= g.N) break;
        y[(int64_t)m * g.ldy + n + k] = (uint16_t)(w0[k >> 1] >> (16 * (k & 1)));
        if (second) y[(int64_t)(m + 1) * g.ldy + n + k] = (uint16_t)(w1[k >> 1] >> (16 * (k & 1)));
      }
    }
  }
}

// Workgroups [0, tiles_big) compute 256 x 256 tiles over columns [0, n_split); the rest
// compute 128 x 128 tiles over columns [n_split, N).  Peeling the last tile columns into
// small tiles keeps the final dispatch round from running a few large tiles on a mostly
// idle GPU.
template <int EPI>
__global__ __launch_bounds__(kPrefillThreads, 1) void gemm_prefill_kernel(GemmArgs g, int n_split, int tiles_big) {
  extern __shared__ __align__(16) uint8_t lds[];
  if ((int)blockIdx.x < tiles_big) {
    int tm, tn;
    tile_coords(blockIdx.x, (g.M + 255) / 256, (n_split + 255) / 256, tm, tn);
    prefill_tile<256, EPI>(g, lds, tm * 256, tn * 256);
  } else {
    int tm, tn;
    tile_coords(blockIdx.x - tiles_big, (g.M + 127) / 128, (g.N - n_split + 127) / 128, tm, tn);
    prefill_tile<128, EPI>(g, lds, tm * 128, n_split + tn * 128);
  }
}

// The same tiling with MXFP4 operands (scaled FP4 MFMAs), fp32 or bf16 output.
__global__ __launch_bounds__(kPrefillThreads, 1) void gemm_mx_kernel(GemmArgs g, int n_split, int tiles_big) {
  extern __shared__ __align__(16) uint8_t lds[];
  if ((int)blockIdx.x < tiles_big) {
    int tm, tn;
    tile_coords(blockIdx.x, (g.M + 255) / 256, (n_split + 255) / 256, tm, tn);
    prefill_tile<256, kEpiStore, true>(g, lds, tm * 256, tn * 256);
  } else {
    int tm, tn;
    tile_coords(blockIdx.x - tiles_big, (g.M + 127) / 128, (g.N - n_split + 127) / 128, tm, tn);
    prefill_tile<128, kEpiStore, true>(g, lds, tm * 128, n_split + tn * 128);
  }
}

// ------------------------------------------------------------------ MXFP4 decode kernel

// M <= 16 tokens on MXFP4 operands: workgroup x owns W rows [32x, 32x + 32) (one 32-row scaled
// MFMA group) and the whole K range; wavefront w takes the 256-wide K stages w, w + 4, ...,
// keeping 4 stages of loads in flight per lane, and the 4 wavefronts' 32 x 32 tiles are summed
// through LDS in a fixed order.  Lane (r, h) = (lane % 32, lane / 32) of a stage loads the 64
// contiguous bytes of codes of MX blocks 4h .. 4h+3 of its A row and W row, and the 4 E8M0
// bytes of those blocks (one dword each); chunk c of the stage multiplies block 4h + c.  The
// same assignment of blocks to (chunk, lane half) holds for A and W, so every dot product is
// unchanged.  Token rows past M load row M - 1 (their outputs are not stored).
struct MxDecodeStage {
  uint4 a[4], w[4];
  uint32_t as, ws;
};

__device__ __forceinline__ void mx_decode_load(const uint8_t* ac, const uint8_t* asc, const uint8_t* wc,
                                               const uint8_t* wsc, int st, MxDecodeStage& d) {
#pragma unroll
  for (int c = 0; c < 4; ++c) d.w[c] = *reinterpret_cast<const uint4*>(wc + st * 128 + 16 * c);
  d.ws = *reinterpret_cast<const uint32_t*>(wsc + st * 8);
#pragma unroll
  for (int c = 0; c < 4; ++c) d.a[c] = *reinterpret_cast<const uint4*>(ac + st * 128 + 16 * c);
  d.as = *reinterpret_cast<const uint32_t*>(asc + st * 8);
}

// Scale byte c of the dwords goes in as byte 0 (the dwords are shifted at their use).
__device__ __forceinline__ void mx_decode_mma(const MxDecodeStage& d, f32x16_t& acc) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(d.a[c]), fp4_operand(d.w[c]), acc, 4, 4, 0,
                                                          (int)(d.as >> (8 * c)), 0, (int)(d.ws >> (8 * c)));
}

constexpr int kMxDecodeThreads = 256;
constexpr int kMxDecodeWaves = kMxDecodeThreads / 64;
constexpr int kMxDecodeRows = 32;

__global__ __launch_bounds__(kMxDecodeThreads) void gemm_mx_decode_kernel(GemmArgs g) {
  __shared__ f32x16_t red[kMxDecodeWaves * 64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * kMxDecodeRows;
  const int64_t kb = (int64_t)g.K / 2, kx = (int64_t)g.K / 32;
  const int nst = g.K / 256;
  const int cnt = wave < nst ? (nst - wave + kMxDecodeWaves - 1) / kMxDecodeWaves : 0;   // this wave's stages
  const int wr = min(n0 + r, g.N - 1), ar = min(r, g.M - 1);
  const uint8_t* ac = g.a_codes + ar * kb + 64 * h;
  const uint8_t* asc = g.a_scales + ar * kx + 4 * h;
  const uint8_t* wc = g.w_codes + wr * kb + 64 * h;
  const uint8_t* wsc = g.w_scales + wr * kx + 4 * h;

  // Stage i is multiplied while i+1 .. i+3 are loading; indices past the wave's last stage
  // reload that stage (a cache hit), unused.
  f32x16_t acc = f32x16_t{};
  if (cnt > 0) {
    const int last = wave + kMxDecodeWaves * (cnt - 1);
    auto st = [&](int i) { return min(wave + kMxDecodeWaves * i, last); };
    MxDecodeStage q0, q1, q2, q3;
    mx_decode_load(ac, asc, wc, wsc, st(0), q0);
    mx_decode_load(ac, asc, wc, wsc, st(1), q1);
    mx_decode_load(ac, asc, wc, wsc, st(2), q2);
    mx_decode_load(ac, asc, wc, wsc, st(3), q3);
    int i = 0;
    for (; i + 4 <= cnt; i += 4) {
      mx_decode_mma(q0, acc);
      __builtin_amdgcn_sched_barrier(0);
      mx_decode_load(ac, asc, wc, wsc, st(i + 4), q0);
      __builtin_amdgcn_sched_barrier(0);
      mx_decode_mma(q1, acc);
      __builtin_amdgcn_sched_barrier(0);
      mx_decode_load(ac, asc, wc, wsc, st(i + 5), q1);
      __builtin_amdgcn_sched_barrier(0);
      mx_decode_mma(q2, acc);
      __builtin_amdgcn_sched_barrier(0);
      mx_decode_load(ac, asc, wc, wsc, st(i + 6), q2);
      __builtin_amdgcn_sched_barrier(0);
      mx_decode_mma(q3, acc);
      __builtin_amdgcn_sched_barrier(0);
      mx_decode_load(ac, asc, wc, wsc, st(i + 7), q3);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int left = cnt - i;
    if (left > 0) mx_decode_mma(q0, acc);
    if (left > 1) mx_decode_mma(q1, acc);
    if (left > 2) mx_decode_mma(q2, acc);
  }
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0) {
    // D[m][n] of the 32 x 32 tile sits in lane n + 32 (m / 4 % 2), register 4 (m / 8) + m % 4;
    // tokens m < 16 are registers 0 .. 7.
    f32x16_t sum = red[lane];
    for (int w = 1; w < kMxDecodeWaves; ++w) sum += red[w * 64 + lane];
    const int n = n0 + r;
    if (n < g.N) {
      const float sw = w_global_at(g, n);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int m = 8 * (q >> 2) + 4 * h + (q & 3);
        if (m < g.M) store_out(g, m, n, (sum[q] * g.a_global[g.a_per_row ? m : 0]) * sw);
      }
    }
  }
}

// ------------------------------------------------------------------ decode kernel

// Operands of one 256-wide K stage for one lane of lane group g = lane / 16: the 32 B of codes
// of K elements [64g, 64g + 64) of the stage and their 4 scale bytes, for A (token row) and
// both W row groups.  The same permutation of K (lane group g takes a contiguous quarter of
// the stage) applies to both operands, so every dot product is unchanged.
struct DecodeStage {
  uint4 a0, a1, w00, w01, w10, w11;
  uint32_t as, ws0, ws1;
};

// Unconditional loads (no branch around any of them), so that the compiler's wait counts
// stay exact and the stages in flight are waited for one at a time.
__device__ __forceinline__ void decode_stage_load(const uint8_t* ac, const uint8_t* asc, const uint8_t* wc0,
                                                  const uint8_t* wsc0, const uint8_t* wc1, const uint8_t* wsc1,
                                                  int st, DecodeStage& d) {
  d.w00 = *reinterpret_cast<const uint4*>(wc0 + st * 128);
  d.w01 = *reinterpret_cast<const uint4*>(wc0 + st * 128 + 16);
  d.w10 = *reinterpret_cast<const uint4*>(wc1 + st * 128);
  d.w11 = *reinterpret_cast<const uint4*>(wc1 + st * 128 + 16);
  d.ws0 = *reinterpret_cast<const uint32_t*>(wsc0 + st * 16);
  d.ws1 = *reinterpret_cast<const uint32_t*>(wsc1 + st * 16);
  d.a0 = *reinterpret_cast<const uint4*>(ac + st * 128);
  d.a1 = *reinterpret_cast<const uint4*>(ac + st * 128 + 16);
  d.as = *reinterpret_cast<const uint32_t*>(asc + st * 16);
}

// 8 MFMA 16x16x32 steps per W row group; one dequantized A fragment serves both groups.
// Dword s of the lane's 32 B of codes belongs to block s/2 of its quarter: scale byte s/2.
__device__ __forceinline__ void decode_stage_mma(const DecodeStage& d, f32x4_t& acc0, f32x4_t& acc1) {
  const uint32_t sel_lo = 0x0c010c00u, sel_hi = 0x0c030c02u;
  const half2_t pa[2] = {__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, d.as, sel_lo) << 7),
                         __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, d.as, sel_hi) << 7)};
  const half2_t p0[2] = {__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, d.ws0, sel_lo) << 7),
                         __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, d.ws0, sel_hi) << 7)};
  const half2_t p1[2] = {__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, d.ws1, sel_lo) << 7),
                         __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0u, d.ws1, sel_hi) << 7)};
  const uint32_t aw[8] = {d.a0.x, d.a0.y, d.a0.z, d.a0.w, d.a1.x, d.a1.y, d.a1.z, d.a1.w};
  const uint32_t w0[8] = {d.w00.x, d.w00.y, d.w00.z, d.w00.w, d.w01.x, d.w01.y, d.w01.z, d.w01.w};
  const uint32_t w1[8] = {d.w10.x, d.w10.y, d.w10.z, d.w10.w, d.w11.x, d.w11.y, d.w11.z, d.w11.w};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int b = s >> 1;
    const half2_t sa = (b & 1) ? half2_t{pa[b >> 1][1], pa[b >> 1][1]} : half2_t{pa[b >> 1][0], pa[b >> 1][0]};
    const half2_t s0 = (b & 1) ? half2_t{p0[b >> 1][1], p0[b >> 1][1]} : half2_t{p0[b >> 1][0], p0[b >> 1][0]};
    const half2_t s1 = (b & 1) ? half2_t{p1[b >> 1][1], p1[b >> 1][1]} : half2_t{p1[b >> 1][0], p1[b >> 1][0]};
    const half8_t fa = dequant8_f16(aw[s], sa);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, dequant8_f16(w0[s], s0), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, dequant8_f16(w1[s], s1), acc1, 0, 0, 0);
  }
}

// Operands of one 128-wide K chunk (used for a last chunk when K / 128 is odd): lane group g
// takes K elements [32g, 32g + 32) of the chunk, 16 B of codes and 2 scale bytes.
struct DecodeChunk {
  uint4 a, w0, w1;
  uint32_t as, ws0, ws1;
};

__device__ __forceinline__ void decode_chunk_load(const uint8_t* ac, const uint8_t* asc, const uint8_t* wc0,
                                                  const uint8_t* wsc0, const uint8_t* wc1, const uint8_t* wsc1,
                                                  DecodeChunk& d) {
  d.w0 = *reinterpret_cast<const uint4*>(wc0);
  d.w1 = *reinterpret_cast<const uint4*>(wc1);
  d.ws0 = *reinterpret_cast<const uint16_t*>(wsc0);
  d.ws1 = *reinterpret_cast<const uint16_t*>(wsc1);
  d.a = *reinterpret_cast<const uint4*>(ac);
  d.as = *reinterpret_cast<const uint16_t*>(asc);
}

__device__ __forceinline__ void decode_chunk_mma(const DecodeChunk& d, f32x4_t& acc0, f32x4_t& acc1) {
  const half2_t pa0 = pair_of_byte(d.as, 0), pa1 = pair_of_byte(d.as, 1);
  const half2_t p00 = pair_of_byte(d.ws0, 0), p01 = pair_of_byte(d.ws0, 1);
  const half2_t p10 = pair_of_byte(d.ws1, 0), p11 = pair_of_byte(d.ws1, 1);
  const uint32_t aw[4] = {d.a.x, d.a.y, d.a.z, d.a.w};
  const uint32_t w0[4] = {d.w0.x, d.w0.y, d.w0.z, d.w0.w};
  const uint32_t w1[4] = {d.w1.x, d.w1.y, d.w1.z, d.w1.w};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const half8_t fa = dequant8_f16(aw[s], s < 2 ? pa0 : pa1);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, dequant8_f16(w0[s], s < 2 ? p00 : p01), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, dequant8_f16(w1[s], s < 2 ? p10 : p11), acc1, 0, 0, 0);
  }
}

// Epilogue of the decode kernels: the 4 wavefronts' 16x16 tiles (red[(wave * 2 + group) * 64 +
// lane]) are summed in a fixed order, scaled (y = (sum * s_gA[m]) * s_gW[seg(n)]) and stored for
// the workgroup's rows n < n_end; for
// NVFP4 output the scaled values of the 16 x 32 tile go through qy (16 x 32 floats of LDS) and
// each of the first 32 threads encodes one 16-column block; with SwiGLU pairs (the workgroup's
// 32 rows are one gate/up pair) each of the first 16 threads takes one token's pair.  GATES:
// gate columns also get their gates from the same fp32 value.
constexpr int kDecodeRowsE = 32;
template <bool GATES>
__device__ __forceinline__ void decode_epilogue(const GemmArgs& g, const f32x4_t* red, float* qy, int wave, int lane,
                                                int n0, int n_end) {
  const int rr = lane & 15, grp = lane >> 4;
  __syncthreads();
  if (wave < 2) {
    // D[m][n] of a 16x16 tile sits in lane n + 16 (m / 4), register m % 4.
    f32x4_t sum = f32x4_t{};
    for (int w = 0; w < 4; ++w) sum += red[(w * 2 + wave) * 64 + lane];
    const int n = n0 + 16 * wave + rr;
    const float sw = n < n_end ? w_global_at(g, n) : 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 4 * grp + q;
      const float v = m < g.M && n < n_end ? (sum[q] * g.a_global[g.a_per_row ? m : 0]) * sw : 0.0f;
      if (g.q_out || g.swiglu)
        qy[m * kDecodeRowsE + 16 * wave + rr] = v;
      else if (m < g.M && n < n_end)
        store_out(g, m, n, v);
      if constexpr (GATES) {
        if (m < g.M && n < n_end && n >= g.gate_n0) store_gate(g, m, n, v);
      }
    }
  }
  if (g.swiglu) {
    __syncthreads();
    const int m = (int)threadIdx.x;
    if (m < 16 && m < g.M && n0 < n_end) store_swiglu_block(g, m, n0, qy + m * kDecodeRowsE, qy + m * kDecodeRowsE + 16);
  } else if (g.q_out) {
    __syncthreads();
    const int t = (int)threadIdx.x;
    if (t < 32) {
      const int m = t >> 1, n = n0 + 16 * (t & 1);
      if (m < g.M && n < n_end) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = qy[m * kDecodeRowsE + 16 * (t & 1) + e];
        store_block_nvfp4(g, m, n, v);
      }
    }
  }
}

// M <= 16 tokens: memory-bound streaming of W in one launch.  Workgroup x owns W rows
// [32x, 32x + 32) (two 16-row MFMA groups) and the whole K range; wavefront w takes the
// 256-wide K stages w, w + 4, w + 8, ... (so a workgroup's loads in flight cover contiguous
// bytes of each row; the last wavefront also takes a final 128-wide chunk), keeps
// kDecodeDepth stages of loads in flight per lane, and the 4 wavefronts reduce their 16x16
// tiles (token x W row) through LDS in a fixed order before the global scales are applied
// and Y is stored.  Token rows past M load row M - 1 (their outputs are not stored).
constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / 64;
constexpr int kDecodeRows = 32;             // W rows per workgroup: two 16-row MFMA groups
constexpr int kDecodeDepth = 4;             // 256-wide stages in flight per lane

template <bool GATES>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_kernel(GemmArgs g) {
  __shared__ f32x4_t red[kDecodeWaves * 2 * 64];
  __shared__ __align__(16) float qy[16 * kDecodeRows];
  // wave is uniform: made explicit so that the stage loop's exits are scalar branches.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rr = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * kDecodeRows;
  const int64_t kb = (int64_t)g.K / 2, ks = (int64_t)g.K / 16;
  const int nchunks = g.K / 128, nst = nchunks / 2;
  const int cnt = wave < nst ? (nst - wave + kDecodeWaves - 1) / kDecodeWaves : 0;   // this wave's stages

  const int wr0 = min(n0 + rr, g.N - 1), wr1 = min(n0 + 16 + rr, g.N - 1);
  const int ar = min(rr, g.M - 1);
  const uint8_t* ac = g.a_codes + ar * kb + grp * 32;
  const uint8_t* asc = g.a_scales + ar * ks + grp * 4;
  const uint8_t* wc0 = g.w_codes + wr0 * kb + grp * 32;
  const uint8_t* wsc0 = g.w_scales + wr0 * ks + grp * 4;
  const uint8_t* wc1 = g.w_codes + wr1 * kb + grp * 32;
  const uint8_t* wsc1 = g.w_scales + wr1 * ks + grp * 4;

  // kDecodeDepth stages in flight per lane: the i-th stage is multiplied while i+1..i+3 are
  // loading.  Indices past the wave's last stage reload that stage (a cache hit), unused:
  // up to 4 such reloads per wavefront.
  f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
  if (cnt > 0) {
    const int last = wave + kDecodeWaves * (cnt - 1);
    auto st = [&](int i) { return min(wave + kDecodeWaves * i, last); };
    DecodeStage q0, q1, q2, q3;
    decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(0), q0);
    decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(1), q1);
    decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(2), q2);
    decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(3), q3);
    // Whole groups of 4 stages (no exit inside, so every load is issued where it stands),
    // then the 0..3 stages left, already loaded.
    int i = 0;
    // The scheduling barriers keep each stage's loads after the multiply that frees its
    // registers and before the next one: hoisted loads would make the in-order wait for the
    // oldest stage also wait for the newest.
    for (; i + kDecodeDepth <= cnt; i += kDecodeDepth) {
      decode_stage_mma(q0, acc0, acc1);
      __builtin_amdgcn_sched_barrier(0);
      decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(i + 4), q0);
      __builtin_amdgcn_sched_barrier(0);
      decode_stage_mma(q1, acc0, acc1);
      __builtin_amdgcn_sched_barrier(0);
      decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(i + 5), q1);
      __builtin_amdgcn_sched_barrier(0);
      decode_stage_mma(q2, acc0, acc1);
      __builtin_amdgcn_sched_barrier(0);
      decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(i + 6), q2);
      __builtin_amdgcn_sched_barrier(0);
      decode_stage_mma(q3, acc0, acc1);
      __builtin_amdgcn_sched_barrier(0);
      decode_stage_load(ac, asc, wc0, wsc0, wc1, wsc1, st(i + 7), q3);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int left = cnt - i;
    if (left > 0) decode_stage_mma(q0, acc0, acc1);
    if (left > 1) decode_stage_mma(q1, acc0, acc1);
    if (left > 2) decode_stage_mma(q2, acc0, acc1);
  }
  if ((nchunks & 1) && wave == kDecodeWaves - 1) {
    const int c = nchunks - 1;   // last 128-wide chunk: lane group g takes its 16 B at g * 16
    DecodeChunk d;
    decode_chunk_load(g.a_codes + ar * kb + c * 64 + grp * 16, g.a_scales + ar * ks + c * 8 + grp * 2,
                      g.w_codes + wr0 * kb + c * 64 + grp * 16, g.w_scales + wr0 * ks + c * 8 + grp * 2,
                      g.w_codes + wr1 * kb + c * 64 + grp * 16, g.w_scales + wr1 * ks + c * 8 + grp * 2, d);
    decode_chunk_mma(d, acc0, acc1);
  }
  red[(wave * 2 + 0) * 64 + lane] = acc0;
  red[(wave * 2 + 1) * 64 + lane] = acc1;
  decode_epilogue<GATES>(g, red, qy, wave, lane, n0, g.N);
}

// M <= 16 tokens, K a multiple of 256: the work of gemm_decode_kernel for a workgroup of
// rows_per_wg <= 32 W rows (rows past the workgroup's last row load that row, their outputs
// are not stored), but every load is a whole 128-byte line copied straight into LDS (8 rows x
// 128 B per wavefront instruction), which moves the same bytes with a third of the memory
// requests of the register loads (16 rows x 64 B, and 16-byte scale pieces).  Each wavefront
// owns a private LDS region: a ring of kDlDepth stages (codes of the 32-row W list and 16
// token rows of one 256-wide K stage) and two blocks of scale bytes (8 stages each); it waits
// for its own copies with explicit counts, so no barrier is needed until the final
// reduction.  Inside a 1 KB chunk of 8 rows, 16-byte piece p of row i sits in slot p ^ i.
constexpr int kDlDepth = 4;                         // 256-wide stages in flight per wavefront
constexpr int kDlChunks = 6;                        // 1 KB chunks: W rows 0-31, then token rows 0-15
constexpr int kDlStageBytes = kDlChunks * 1024;     // codes of one stage
constexpr int kDlScaleBytes = kDlChunks * 1024;     // scale bytes of 8 stages
constexpr int kDlWaveBytes = kDlDepth * kDlStageBytes + 2 * kDlScaleBytes;
constexpr int kDlRedOffset = kDecodeWaves * kDlWaveBytes;
constexpr int kDlLds = kDlRedOffset + kDecodeWaves * 2 * 64 * 16;

// s_waitcnt immediate that waits for at most n outstanding vector memory operations.
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

__device__ __forceinline__ int dl_slot(int i, int p) { return i * 128 + ((p ^ i) << 4); }

// Copies for one chunk: 8 rows (row_of(i) -> byte offset of that row from base) x 128 B at col.
__device__ __forceinline__ void dl_copy_chunk(const uint8_t* base, uint32_t row_off, uint32_t col, int lane,
                                              const uint8_t* dst) {
  const int i = lane >> 3, p = (lane & 7) ^ i;
  copy16_to_lds(base, row_off + col + p * 16, dst);
}

template <int WC, int TC, bool GATES>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_lds_kernel(GemmArgs g, int rows_per_wg) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rr = lane & 15, grp = lane >> 4, i8 = lane >> 3;
  const int n0 = blockIdx.x * rows_per_wg;              // rows [n0, n_end), at most 32
  const int n_end = min(n0 + rows_per_wg, g.N);
  const uint32_t kb = (uint32_t)g.K / 2, ks = (uint32_t)g.K / 16;
  const int nst = g.K / 256;
  const int s0 = wave * nst / kDecodeWaves, cnt = (wave + 1) * nst / kDecodeWaves - s0;
  uint8_t* region = lds + wave * kDlWaveBytes;

  // Only the chunks that hold real rows are copied: W chunks 0 .. WC - 1 (WC = ceil(rows / 8))
  // and token chunks 4 .. 3 + TC (TC = ceil(M / 8)), NC copies per stage and per scale block.
  // The multiplies below read every chunk; what a chunk that is not copied holds reaches only
  // the outputs of padding rows and tokens, which are never stored.  Per-lane row offsets of the
  // rows this lane copies (row i8 of each chunk), clamped.
  constexpr int NC = WC + TC;
  auto chunk_of = [](int c) { return c < WC ? c : 4 + (c - WC); };
  uint32_t row_codes[NC], row_scales[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int r = c < WC ? min(8 * c + i8, n_end - 1 - n0) : min(8 * (c - WC) + i8, g.M - 1);
    row_codes[c] = (uint32_t)r * kb;
    row_scales[c] = (uint32_t)r * ks;
  }
  const uint8_t* wcb = g.w_codes + (size_t)n0 * kb;
  const uint8_t* wsb = g.w_scales + (size_t)n0 * ks;
  const uint32_t last_piece = ks - 16;
  auto copy_codes = [&](int t) {      // stage t of this wavefront (clamped to its last)
    const uint32_t col = (uint32_t)(s0 + min(t, cnt - 1)) * 128;
    uint8_t* dst = region + (t % kDlDepth) * kDlStageBytes;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      dl_copy_chunk(c < WC ? wcb : g.a_codes, row_codes[c], col, lane, dst + chunk_of(c) * 1024);
  };
  auto copy_scales = [&](int b) {     // scale bytes of stages 8b .. 8b + 7 of this wavefront
    const uint32_t col = (uint32_t)(s0 + 8 * b) * 16;
    uint8_t* dst = region + kDlDepth * kDlStageBytes + (b & 1) * kDlScaleBytes;
    const uint32_t p16 = (uint32_t)(((lane & 7) ^ i8) * 16);
#pragma unroll
    for (int c = 0; c < NC; ++c)   // pieces past the row's end (never read) clamped in bounds
      copy16_to_lds(c < WC ? wsb : g.a_scales, row_scales[c] + min(col + p16, last_piece),
                    dst + chunk_of(c) * 1024);
  };

  f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
  if (cnt > 0) {
    copy_scales(0);
#pragma unroll
    for (int t = 0; t < kDlDepth; ++t) copy_codes(t);
    const int iw = rr & 7;
    for (int t = 0; t < cnt; ++t) {
      // Stage t's copies (and its scale block) are older than the NC (kDlDepth - 1) copies of
      // the next stages: at most that many may still be in flight.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NC * (kDlDepth - 1)));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* cs = region + (t % kDlDepth) * kDlStageBytes;
      const uint8_t* ss = region + kDlDepth * kDlStageBytes + ((t >> 3) & 1) * kDlScaleBytes;
      const int q = t & 7;
      const int c0 = rr >> 3;               // chunk of W row rr (group 0); +2 for group 1; +4 tokens
      DecodeStage d;
      d.w00 = *reinterpret_cast<const uint4*>(cs + c0 * 1024 + dl_slot(iw, 2 * grp));
      d.w01 = *reinterpret_cast<const uint4*>(cs + c0 * 1024 + dl_slot(iw, 2 * grp + 1));
      d.w10 = *reinterpret_cast<const uint4*>(cs + (c0 + 2) * 1024 + dl_slot(iw, 2 * grp));
      d.w11 = *reinterpret_cast<const uint4*>(cs + (c0 + 2) * 1024 + dl_slot(iw, 2 * grp + 1));
      d.a0 = *reinterpret_cast<const uint4*>(cs + (c0 + 4) * 1024 + dl_slot(iw, 2 * grp));
      d.a1 = *reinterpret_cast<const uint4*>(cs + (c0 + 4) * 1024 + dl_slot(iw, 2 * grp + 1));
      d.ws0 = *reinterpret_cast<const uint32_t*>(ss + c0 * 1024 + dl_slot(iw, q) + 4 * grp);
      d.ws1 = *reinterpret_cast<const uint32_t*>(ss + (c0 + 2) * 1024 + dl_slot(iw, q) + 4 * grp);
      d.as = *reinterpret_cast<const uint32_t*>(ss + (c0 + 4) * 1024 + dl_slot(iw, q) + 4 * grp);
      decode_stage_mma(d, acc0, acc1);
      __builtin_amdgcn_sched_barrier(0);
      // The slot just read is refilled with stage t + kDlDepth (its reads are complete: the
      // MFMAs above consumed them); a scale block is refilled once its 8 stages are done.
      copy_codes(t + kDlDepth);
      if (((t + kDlDepth) & 7) == 0) copy_scales((t + kDlDepth) >> 3);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + kDlRedOffset);
  red[(wave * 2 + 0) * 64 + lane] = acc0;
  red[(wave * 2 + 1) * 64 + lane] = acc1;
  decode_epilogue<GATES>(g, red, reinterpret_cast<float*>(lds), wave, lane, n0, n_end);
}

// M <= 4 tokens and at most 20 rows per workgroup: the K-split scheme above (the same LDS ring
// layout and copies, minus the chunks of padding rows), multiplied with the 16-block 4 x 4 x 4 fp16
// MFMA instead of 16 x 16 x 32, so that no padding row is dequantized: the workgroup's rows go in
// NG groups of 4 (4 NG >= rows) and the tokens in one group of 4.  Block b of an instruction takes
// K elements [16b + 4f, 16b + 4f + 4) of the stage (f = 0..3 over four instructions), so lane 4b +
// i dequantizes exactly one 16-element block (8 B of codes, one scale byte) of W row 4g + i per
// group and stage, and lane 4b + j one block of token j, which serves all NG groups.  A and W take
// the same K order, so every dot product is unchanged.  D of block b sits in lane 4b + j, register
// i (W row i, token j); the 16 blocks' partial sums are added once after the loop: two DPP
// rotations within each row of 16 lanes, then the four row sums through LDS, in a fixed order.
// This instruction issues far less work per cycle than 16 x 16 x 32, so it pays only while the
// dequantization it saves dominates: more tokens or rows take gemm_decode_lds_kernel.
template <int NG, bool GATES>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_q4_kernel(GemmArgs g, int rows_per_wg) {
  constexpr int NT = 1;
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int i8 = lane >> 3;
  const int n0 = blockIdx.x * rows_per_wg;              // rows [n0, n_end), at most 4 NG <= 32
  const int n_end = min(n0 + rows_per_wg, g.N);
  const uint32_t kb = (uint32_t)g.K / 2, ks = (uint32_t)g.K / 16;
  const int nst = g.K / 256;
  const int s0 = wave * nst / kDecodeWaves, cnt = (wave + 1) * nst / kDecodeWaves - s0;
  uint8_t* region = lds + wave * kDlWaveBytes;

  // The ring layout of gemm_decode_lds_kernel (chunk c of a stage at c KB: W rows 8c .. 8c + 7
  // for c < 4, token rows 0-7 in chunk 4), but only the chunks this kernel reads are copied: the
  // W chunks of rows 0 .. 4 NG - 1 and token chunk 4 (rows past the workgroup's last row or
  // past M load that last row).  NC copies per stage and per scale block.
  constexpr int kWChunks = (4 * NG + 7) / 8, NC = kWChunks + 1;
  auto chunk_of = [](int c) { return c < kWChunks ? c : 4; };
  uint32_t row_codes[NC], row_scales[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int r = c < kWChunks ? min(8 * c + i8, n_end - 1 - n0) : min(i8, g.M - 1);
    row_codes[c] = (uint32_t)r * kb;
    row_scales[c] = (uint32_t)r * ks;
  }
  const uint8_t* wcb = g.w_codes + (size_t)n0 * kb;
  const uint8_t* wsb = g.w_scales + (size_t)n0 * ks;
  const uint32_t last_piece = ks - 16;
  auto copy_codes = [&](int t) {
    const uint32_t col = (uint32_t)(s0 + min(t, cnt - 1)) * 128;
    uint8_t* dst = region + (t % kDlDepth) * kDlStageBytes;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      dl_copy_chunk(c < kWChunks ? wcb : g.a_codes, row_codes[c], col, lane, dst + chunk_of(c) * 1024);
  };
  auto copy_scales = [&](int b) {
    const uint32_t col = (uint32_t)(s0 + 8 * b) * 16;
    uint8_t* dst = region + kDlDepth * kDlStageBytes + (b & 1) * kDlScaleBytes;
    const uint32_t p16 = (uint32_t)(((lane & 7) ^ i8) * 16);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      copy16_to_lds(c < kWChunks ? wsb : g.a_scales, row_scales[c] + min(col + p16, last_piece),
                    dst + chunk_of(c) * 1024);
  };

  // Lane 4b + i: block b of the stage (16 B piece b / 2 of a row, its half b % 2), row i of a
  // group.  Row r of the ring (W rows 0-31, then token m as row 32 + m) is row r % 8 of chunk
  // r / 8.
  const int bq = lane >> 2, iq = lane & 3;
  const int piece = bq >> 1, half_off = (bq & 1) * 8;
  f32x4_t acc[NG][NT];
#pragma unroll
  for (int a = 0; a < NG; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f32x4_t{};
  if (cnt > 0) {
    copy_scales(0);
#pragma unroll
    for (int t = 0; t < kDlDepth; ++t) copy_codes(t);
    for (int t = 0; t < cnt; ++t) {
      // Stage t's copies and its scale block are older than the NC (kDlDepth - 1) copies of the
      // next stages.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NC * (kDlDepth - 1)));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* cs = region + (t % kDlDepth) * kDlStageBytes;
      const uint8_t* ss = region + kDlDepth * kDlStageBytes + ((t >> 3) & 1) * kDlScaleBytes;
      const int q = t & 7;
      // The lane's block of ring row r, dequantized: fragment f holds its K elements [4f, 4f + 4).
      auto block_frags = [&](int r, half4_t (&f)[4]) {
        const uint2 c = *reinterpret_cast<const uint2*>(cs + (r >> 3) * 1024 + dl_slot(r & 7, piece) + half_off);
        uint32_t u = (uint32_t)ss[(r >> 3) * 1024 + dl_slot(r & 7, q) + bq] << 7;   // E4M3 * 2^-8 as fp16
        u |= u << 16;
        const half2_t sc = __builtin_bit_cast(half2_t, u);
        const half8_t lo = dequant8_f16(c.x, sc), hi = dequant8_f16(c.y, sc);
        f[0] = __builtin_shufflevector(lo, lo, 0, 1, 2, 3);
        f[1] = __builtin_shufflevector(lo, lo, 4, 5, 6, 7);
        f[2] = __builtin_shufflevector(hi, hi, 0, 1, 2, 3);
        f[3] = __builtin_shufflevector(hi, hi, 4, 5, 6, 7);
      };
      half4_t tf[NT][4];
#pragma unroll
      for (int b = 0; b < NT; ++b) block_frags(32 + 4 * b + iq, tf[b]);
#pragma unroll
      for (int a = 0; a < NG; ++a) {
        half4_t wf[4];
        block_frags(4 * a + iq, wf);
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
          for (int f = 0; f < 4; ++f) acc[a][b] = __builtin_amdgcn_mfma_f32_4x4x4f16(wf[f], tf[b][f], acc[a][b], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      copy_codes(t + kDlDepth);
      if (((t + kDlDepth) & 7) == 0) copy_scales((t + kDlDepth) >> 3);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  // Sum over the blocks within each row of 16 lanes (lanes 4b + j, b = 4R .. 4R + 3): after the
  // rotations by 4 and 8 every lane of row R holds that row's sum for its token j.  Lanes 16R + j
  // (j < 4) leave the row sums in this wavefront's ring region: part[(a NT + b) 4 + i][4R + j].
  float* part = reinterpret_cast<float*>(region);
#pragma unroll
  for (int a = 0; a < NG; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[a][b][i];
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true));   // row_ror:4
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));   // row_ror:8
        if ((lane & 15) < 4) part[((a * NT + b) * 4 + i) * 16 + (lane >> 4) * 4 + (lane & 3)] = v;
      }
  __syncthreads();
  // The wavefront's 16 x 16 tiles in the layout the epilogue reads (W row n of group G, token m
  // in lane n + 16 (m / 4), register m % 4): lane l takes n = l % 16 and token group l / 16.
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + kDlRedOffset);
#pragma unroll
  for (int G = 0; G < 2; ++G) {
    const int r = 16 * G + (lane & 15), tg = lane >> 4;
    const int a = r >> 2, i = r & 3;
    f32x4_t s = f32x4_t{};
    if (a < NG && tg < NT) {
      const f32x4_t* p = reinterpret_cast<const f32x4_t*>(part + ((a * NT + tg) * 4 + i) * 16);
      s = ((p[0] + p[1]) + p[2]) + p[3];
    }
    red[(wave * 2 + G) * 64 + lane] = s;
  }
  decode_epilogue<GATES>(g, red, reinterpret_cast<float*>(lds), wave, lane, n0, n_end);
}

// The instantiation of gemm_decode_lds_kernel that copies WC W chunks (2 to 4: 16 to 32 rows) and
// TC token chunks (1 or 2: up to 8 or 16 tokens).
typedef void (*DecodeLdsKernel)(GemmArgs, int);
DecodeLdsKernel decode_lds_kernel(bool gated, int wc, int tc) {
  static constexpr DecodeLdsKernel k[2][3][2] = {
      {{gemm_decode_lds_kernel<2, 1, false>, gemm_decode_lds_kernel<2, 2, false>},
       {gemm_decode_lds_kernel<3, 1, false>, gemm_decode_lds_kernel<3, 2, false>},
       {gemm_decode_lds_kernel<4, 1, false>, gemm_decode_lds_kernel<4, 2, false>}},
      {{gemm_decode_lds_kernel<2, 1, true>, gemm_decode_lds_kernel<2, 2, true>},
       {gemm_decode_lds_kernel<3, 1, true>, gemm_decode_lds_kernel<3, 2, true>},
       {gemm_decode_lds_kernel<4, 1, true>, gemm_decode_lds_kernel<4, 2, true>}}};
  return k[gated][wc - 2][tc - 1];
}

// M <= 16 tokens on MXFP4 operands with K a multiple of 512: the K-split scheme above (each
// wavefront copies and multiplies its own contiguous range of 256-wide stages through a
// private LDS ring: W rows 0-31 in chunks 0-3, token rows 0-15 in chunks 4-5), with the
// scaled FP4 MFMA reading its operands from the ring.  MX scale bytes are 8 per row and
// stage, so one 1 KB scale chunk holds 16 stages of 8 rows (16 B piece p of a row = stages
// 2p and 2p+1); K % 512 == 0 and an even first stage per wavefront keep every piece whole and
// 16-byte aligned.  Lane (r, h) multiplies MX block 4h + c of the stage in chunk c for W row r
// and token row r mod 16 (lanes 16-31 read the same LDS rows as 0-15; their outputs are not
// stored), with the stage's scale dword at byte 4h of its 8.
template <int WC, int TC>
__global__ __launch_bounds__(kDecodeThreads) void gemm_mx_decode_lds_kernel(GemmArgs g, int rows_per_wg) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int i8 = lane >> 3, r = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * rows_per_wg;              // rows [n0, n_end), at most 32
  const int n_end = min(n0 + rows_per_wg, g.N);
  const uint32_t kb = (uint32_t)g.K / 2, kx = (uint32_t)g.K / 32;
  const int pairs = g.K / 512;
  const int s0 = 2 * (wave * pairs / kDecodeWaves), cnt = 2 * ((wave + 1) * pairs / kDecodeWaves) - s0;
  uint8_t* region = lds + wave * kDlWaveBytes;

  // As in gemm_decode_lds_kernel, only the chunks that hold real rows are copied: W chunks
  // 0 .. WC - 1 and token chunks 4 .. 3 + TC, NC copies per stage and per scale block; the
  // multiplies read every chunk, and what an uncopied chunk holds reaches only outputs that are
  // never stored.
  constexpr int NC = WC + TC;
  auto chunk_of = [](int c) { return c < WC ? c : 4 + (c - WC); };
  uint32_t row_codes[NC], row_scales[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int rw = c < WC ? min(8 * c + i8, n_end - 1 - n0) : min(8 * (c - WC) + i8, g.M - 1);
    row_codes[c] = (uint32_t)rw * kb;
    row_scales[c] = (uint32_t)rw * kx;
  }
  const uint8_t* wcb = g.w_codes + (size_t)n0 * kb;
  const uint8_t* wxb = g.w_scales + (size_t)n0 * kx;
  const uint32_t last_piece = kx - 16;
  auto copy_codes = [&](int t) {      // stage t of this wavefront (clamped to its last)
    const uint32_t col = (uint32_t)(s0 + min(t, cnt - 1)) * 128;
    uint8_t* dst = region + (t % kDlDepth) * kDlStageBytes;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      dl_copy_chunk(c < WC ? wcb : g.a_codes, row_codes[c], col, lane, dst + chunk_of(c) * 1024);
  };
  auto copy_scales = [&](int b) {     // scale bytes of stages 16b .. 16b + 15 of this wavefront
    const uint32_t col = (uint32_t)(s0 + 16 * b) * 8;
    uint8_t* dst = region + kDlDepth * kDlStageBytes + (b & 1) * kDlScaleBytes;
    const uint32_t p16 = (uint32_t)(((lane & 7) ^ i8) * 16);
#pragma unroll
    for (int c = 0; c < NC; ++c)   // pieces past the row's end (never read) clamped in bounds
      copy16_to_lds(c < WC ? wxb : g.a_scales, row_scales[c] + min(col + p16, last_piece),
                    dst + chunk_of(c) * 1024);
  };

  f32x16_t acc = f32x16_t{};
  if (cnt > 0) {
    copy_scales(0);
#pragma unroll
    for (int t = 0; t < kDlDepth; ++t) copy_codes(t);
    const int iw = r & 7, wch = r >> 3, ach = 4 + ((r & 15) >> 3);
    for (int t = 0; t < cnt; ++t) {
      // Stage t's copies (and its scale block) are older than the NC (kDlDepth - 1) copies of
      // the next stages: at most that many may still be in flight.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NC * (kDlDepth - 1)));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* cs = region + (t % kDlDepth) * kDlStageBytes;
      const uint8_t* ss = region + kDlDepth * kDlStageBytes + ((t >> 4) & 1) * kDlScaleBytes;
      const int sp = dl_slot(iw, (t & 15) >> 1) + 8 * (t & 1) + 4 * h;
      const uint32_t ws = *reinterpret_cast<const uint32_t*>(ss + wch * 1024 + sp);
      const uint32_t as = *reinterpret_cast<const uint32_t*>(ss + ach * 1024 + sp);
      uint4 w[4], a[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        w[c] = *reinterpret_cast<const uint4*>(cs + wch * 1024 + dl_slot(iw, 4 * h + c));
        a[c] = *reinterpret_cast<const uint4*>(cs + ach * 1024 + dl_slot(iw, 4 * h + c));
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(a[c]), fp4_operand(w[c]), acc, 4, 4, 0,
                                                              (int)(as >> (8 * c)), 0, (int)(ws >> (8 * c)));
      __builtin_amdgcn_sched_barrier(0);
      // The slot just read is refilled with stage t + kDlDepth; a scale block is refilled
      // once its 16 stages are done.  The MFMAs may be scheduled after the refill copies, so
      // the stage's LDS reads are waited for here, before any copy can overwrite them.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
      copy_codes(t + kDlDepth);
      if (((t + kDlDepth) & 15) == 0) copy_scales((t + kDlDepth) >> 4);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  __syncthreads();              // every wavefront is done with its ring: the sum reuses LDS
  f32x16_t* red = reinterpret_cast<f32x16_t*>(lds);
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0) {
    // D[m][n] of the 32 x 32 tile sits in lane n + 32 (m / 4 % 2), register 4 (m / 8) + m % 4;
    // tokens m < 16 are registers 0 .. 7.
    f32x16_t sum = red[lane];
    for (int w = 1; w < kDecodeWaves; ++w) sum += red[w * 64 + lane];
    const int n = n0 + r;
    if (n < n_end) {
      const float sw = w_global_at(g, n);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int m = 8 * (q >> 2) + 4 * h + (q & 3);
        if (m < g.M) store_out(g, m, n, (sum[q] * g.a_global[g.a_per_row ? m : 0]) * sw);
      }
    }
  }
}

// The instantiation of gemm_mx_decode_lds_kernel that copies WC W chunks (2 to 4) and TC token
// chunks (1 or 2).
DecodeLdsKernel mx_decode_lds_kernel(int wc, int tc) {
  static constexpr DecodeLdsKernel k[3][2] = {
      {gemm_mx_decode_lds_kernel<2, 1>, gemm_mx_decode_lds_kernel<2, 2>},
      {gemm_mx_decode_lds_kernel<3, 1>, gemm_mx_decode_lds_kernel<3, 2>},
      {gemm_mx_decode_lds_kernel<4, 1>, gemm_mx_decode_lds_kernel<4, 2>}};
  return k[wc - 2][tc - 1];
}

// ------------------------------------------------------------------ decode, balanced rows

// M <= 16 tokens, K a multiple of 256, one launch in which every CU streams the same bytes:
// workgroup b owns W rows [b R, b R + R) and all of K, R (at most 16 G) chosen by the host so
// that the grid is a whole number of rounds over the CUs (68 rows per workgroup, one round,
// for N = 17408 on 256 CUs).
//
// A 256-wide K stage holds the codes of the 16 G W rows and the 16 token rows as 1 KB chunks
// of 8 rows x 128 B (whole lines; 16-byte piece p of row i in slot p ^ i), copied straight
// from global memory into a ring of kDepth stages shared by the workgroup.  Wavefronts 0-3
// issue the copies, the chunks of a stage shared out among them (a wavefront with fewer
// chunks than the others copies chunk 0 again into a scratch slot, so each issues the same
// number per stage; copying only the chunks that hold real rows measured slower).  The loop
// runs in steps of kSteps stages: at the top of a step every copying wavefront waits for its
// copies of the step's stages, the step's only barrier publishes them to all and frees the
// slots of the previous step, which are refilled at once kDepth - kSteps stages ahead.  kSteps and kDepth grow as the stage shrinks (fewer row
// groups), so every step and the bytes in flight stay large.  The scale bytes of all rows
// over all of K are copied once, up front, in the same chunk layout (8 rows x 8 stages of
// 16 B per chunk).
//
// Eight wavefronts, two per SIMD so that one's dequantization hides the other's waits:
// wavefront w multiplies K elements [32 w, 32 w + 32) of every stage for all G row groups, one
// 16x16x32 MFMA per group (lane group q supplies K elements 32 w + 8 q .. + 8, inside one
// block, so one scale byte) with one dequantized token fragment shared by the groups.  The
// eight partial tiles of a group are summed in a fixed order at the end.  Rows past the
// workgroup's last row load that row and token rows past M load row M - 1; their outputs are
// not stored.
template <int G> struct DwCfg {
  static constexpr int kChunks = 2 * G + 2;             // 1 KB chunks per stage: W rows, then tokens
  static constexpr int kPerWave = (kChunks + 3) / 4;    // copies per copying wavefront per stage
  static constexpr int kStageBytes = kChunks * 1024;
  static constexpr int kSteps = G >= 3 ? 2 : 4;         // stages per barrier
  static constexpr int kDepth = 4 * kSteps;             // stages in the ring
  static constexpr int kScratch = kDepth * kStageBytes; // 1 KB target of padding copies
  static constexpr int kScales = kScratch + 1024;       // scale chunks: block b, chunk c at (b kChunks + c) KB
};
constexpr int kDwMaxG = 5;     // row groups per workgroup; SwiGLU pairs may take kDwPairG
constexpr int kDwPairG = 6;
constexpr int kDwThreads = 512;

// LDS bytes of the balanced decode kernel for G row groups and K (0 if K does not fit).
template <int G>
int dw_lds_bytes_g(int64_t K) {
  using C = DwCfg<G>;
  const int64_t blocks = (K / 256 + 7) / 8;
  const int64_t bytes = C::kScales + blocks * C::kChunks * 1024;
  return bytes <= 160 * 1024 ? (int)bytes : 0;
}
inline int dw_lds_bytes(int G, int64_t K) {
  switch (G) {
    case 1: return dw_lds_bytes_g<1>(K);
    case 2: return dw_lds_bytes_g<2>(K);
    case 3: return dw_lds_bytes_g<3>(K);
    case 4: return dw_lds_bytes_g<4>(K);
    case 5: return dw_lds_bytes_g<5>(K);
    case kDwPairG: return dw_lds_bytes_g<kDwPairG>(K);
    default: return 0;
  }
}

// Copy chunk c (rows 8c .. 8c+7 of the stage's row list) of 256-wide stage t: lane l copies
// 16-byte piece (l & 7) ^ (l >> 3) of row l >> 3 into slot l & 7 of that row.
template <int G>
__device__ __forceinline__ void dw_copy_codes(const GemmArgs& g, const uint8_t* wcb, const uint32_t (&row_off)[DwCfg<G>::kPerWave],
                                              int wave, int lane, int t, uint8_t* lds) {
  using C = DwCfg<G>;
  const uint32_t piece = (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16) + (uint32_t)t * 128;
  uint8_t* stage = lds + (t % C::kDepth) * C::kStageBytes;
#pragma unroll
  for (int i = 0; i < C::kPerWave; ++i) {
    const int c = wave + 4 * i;
    if (c < C::kChunks)
      copy16_to_lds(c < 2 * G ? wcb : g.a_codes, row_off[i] + piece, stage + c * 1024);
    else
      copy16_to_lds(wcb, row_off[i] + piece, lds + C::kScratch);
  }
}

// s_waitcnt for at most n stages of copies (n <= kDepth - 2 kSteps) still in flight.
template <int G>
__device__ __forceinline__ void dw_wait_stages(int n) {
  using C = DwCfg<G>;
  static_assert(C::kDepth - 2 * C::kSteps <= 8 && 8 * C::kPerWave <= 63, "wait cases");
  switch (n) {
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 * C::kPerWave)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7 * C::kPerWave)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * C::kPerWave)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * C::kPerWave)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * C::kPerWave)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * C::kPerWave)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::kPerWave)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1 * C::kPerWave)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
  }
}

template <int G, bool GATES>
__global__ __launch_bounds__(kDwThreads) void gemm_decode_rows_kernel(GemmArgs g, int rows_per_wg) {
  using C = DwCfg<G>;
  constexpr int S = C::kSteps, D = C::kDepth;
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rr = lane & 15, q = lane >> 4;
  const int r0 = blockIdx.x * rows_per_wg;
  const int rw = min(rows_per_wg, g.N - r0);             // rows of this workgroup (>= 1)
  const uint32_t kb = (uint32_t)g.K / 2, ks = (uint32_t)g.K / 16;
  const int nst = g.K / 256;
  const uint8_t* wcb = g.w_codes + (size_t)r0 * kb;
  const uint8_t* wsb = g.w_scales + (size_t)r0 * ks;

  // Row of the stage's row list that lane l copies in chunk c: W row min(8c + l/8, rw - 1) of
  // the workgroup, or token row min(8(c - 2G) + l/8, M - 1); chunks past the list copy row 0.
  auto list_row = [&](int c, uint32_t pitch) -> uint32_t {
    const int i = lane >> 3;
    if (c < 2 * G) return (uint32_t)min(8 * c + i, rw - 1) * pitch;
    if (c < C::kChunks) return (uint32_t)min(8 * (c - 2 * G) + i, g.M - 1) * pitch;
    return 0u;
  };
  const bool copier = wave < 4;
  uint32_t row_off[C::kPerWave];
#pragma unroll
  for (int i = 0; i < C::kPerWave; ++i) row_off[i] = list_row((wave & 3) + 4 * i, kb);

  // Scale bytes, all stages: block b (stages 8b .. 8b+7), chunk c = rows 8c .. 8c+7, each
  // row's 8 pieces of 16 B (one per stage) in the code chunks' slot order; pieces past the
  // last stage repeat it.
  {
    const int nblk = (nst + 7) / 8;
    const int p = (lane & 7) ^ (lane >> 3);
    for (int e = wave; e < nblk * C::kChunks; e += 8) {
      const int b = e / C::kChunks, c = e - b * C::kChunks;
      const uint32_t off = list_row(c, ks) + (uint32_t)min(8 * b + p, nst - 1) * 16;
      copy16_to_lds(c < 2 * G ? wsb : g.a_scales, off, lds + C::kScales + e * 1024);
    }
  }
  if (copier) {
    for (int t = 0; t < D - S && t < nst; ++t) dw_copy_codes<G>(g, wcb, row_off, wave, lane, t, lds);
  } else {
    // The loop's waits count stage copies, which these wavefronts do not issue: their scale
    // copies must be complete before the first barrier.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  // Where this lane reads: row rr & 7 of chunk 2j + rr/8 (W group j) or 2G + rr/8 (tokens),
  // 4 bytes at byte 16 w + 4 q of the row's 128 (piece w), and scale byte 2w + q/2 of the
  // stage's 16 (dword w/2).
  const int ir = rr & 7, ch = rr >> 3;
  const int code_off = ir * 128 + ((wave ^ ir) << 4) + 4 * q;
  const int sc_off = 4 * (wave >> 1);
  const int byte_sh = 8 * (2 * (wave & 1) + (q >> 1));
  f32x4_t acc[G];
#pragma unroll
  for (int j = 0; j < G; ++j) acc[j] = f32x4_t{};

  for (int t0 = 0; t0 < nst; t0 += S) {
    // Stages t0 .. t0+S-1 must be complete; copies issued after them (up to stage
    // t0 + D - S - 1, at most D - 2S stages) may still be in flight.
    dw_wait_stages<G>(min(t0 + D - S - 1, nst - 1) - min(t0 + S - 1, nst - 1));
    asm volatile("" ::: "memory");
    __syncthreads();            // this step's stages copied by every wavefront; the last step's read by all
    if (copier) {
#pragma unroll
      for (int u = 0; u < S; ++u)
        if (t0 + D - S + u < nst) dw_copy_codes<G>(g, wcb, row_off, wave, lane, t0 + D - S + u, lds);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int t = t0 + u;
      if (t < nst) {
        const uint8_t* stage = lds + (t % D) * C::kStageBytes;
        const uint8_t* sc = lds + C::kScales + (t >> 3) * C::kChunks * 1024 + ir * 128 + (((t & 7) ^ ir) << 4) + sc_off;
        const uint32_t a = *reinterpret_cast<const uint32_t*>(stage + (2 * G + ch) * 1024 + code_off);
        const uint32_t as = *reinterpret_cast<const uint32_t*>(sc + (2 * G + ch) * 1024);
        const half8_t fa = dequant8_f16(a, scale_pair_f16((as >> byte_sh) & 0xFFu));
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(stage + (2 * j + ch) * 1024 + code_off);
          const uint32_t ws = *reinterpret_cast<const uint32_t*>(sc + (2 * j + ch) * 1024);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, dequant8_f16(w, scale_pair_f16((ws >> byte_sh) & 0xFFu)),
                                                          acc[j], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Sum the eight wavefronts' tiles of each group in a fixed order, then scale and store.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  __syncthreads();              // every wavefront is done with the ring
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds);
#pragma unroll
  for (int j = 0; j < G; ++j) red[(wave * G + j) * 64 + lane] = acc[j];
  __syncthreads();
  float* qy = reinterpret_cast<float*>(lds + 8 * G * 1024);   // 16 tokens x 16 G columns (NVFP4 out)
  for (int j = wave; j < G; j += 8) {
    // D[m][n] of a 16x16 tile sits in lane n + 16 (m / 4), register m % 4.
    f32x4_t sum = red[j * 64 + lane];
    for (int w = 1; w < 8; ++w) sum += red[(w * G + j) * 64 + lane];
    const int nl = 16 * j + rr, n = r0 + nl;
    const bool nv = nl < rw;
    const float sw = nv ? w_global_at(g, n) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      const bool ok = m < g.M && nv;
      const float v = ok ? (sum[i] * g.a_global[g.a_per_row ? m : 0]) * sw : 0.0f;
      if (g.q_out || g.swiglu)
        qy[m * (16 * G) + nl] = v;
      else if (ok)
        store_out(g, m, n, v);
      if constexpr (GATES) {
        if (ok && n >= g.gate_n0) store_gate(g, m, n, v);
      }
    }
  }
  if (g.swiglu) {
    // Rows per workgroup are a multiple of 32 here, so G is even: G / 2 gate/up pairs (the
    // host never picks an odd G for SwiGLU pairs).
    __syncthreads();
    if constexpr (G % 2 == 0) {
      constexpr int P = G / 2;
      const int t = (int)threadIdx.x;
      if (t < 16 * P) {
        const int m = t / P, j = t - m * P;
        const float* v = qy + m * (16 * G) + 32 * j;
        if (m < g.M && 32 * j < rw) store_swiglu_block(g, m, r0 + 32 * j, v, v + 16);
      }
    }
  } else if (g.q_out) {
    __syncthreads();
    const int t = (int)threadIdx.x;
    if (t < 16 * G) {
      const int m = t / G, j = t - m * G;
      if (m < g.M && 16 * j < rw) {
        float v[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = qy[m * (16 * G) + 16 * j + e];
        store_block_nvfp4(g, m, r0 + 16 * j, v);
      }
    }
  }
}

// ------------------------------------------------------------------ MXFP4 decode, balanced rows

// M <= 16 tokens on MXFP4 operands, N > 32 x CUs, K % 512 == 0: the balanced-rows scheme of
// gemm_decode_rows_kernel with G groups of 32 W rows (one scaled 32 x 32 x 64 MFMA group
// each).  The 8 wavefronts share one ring of kDepth 256-wide stages (wavefronts 0-3 copy,
// kSteps stages per barrier); every scale byte of the workgroup's rows is copied up front.
// Wavefront w multiplies the 64-element piece w % 4 of every stage for the groups w / 4,
// w / 4 + 2, ...: lane (r, h) takes MX block 2 (w % 4) + h of W row r of the group and of token
// row r mod 16.  The 4 wavefronts of a group are summed through LDS in a fixed order.  MX scale
// bytes are 8 per row and stage: a 1 KB scale chunk holds 16 stages of 8 rows (16 B piece q of a
// row = stages 2q, 2q+1), so K % 512 == 0 keeps every piece whole.
template <int G> struct MxDwCfg {
  static constexpr int kChunks = 4 * G + 2;             // 1 KB chunks per stage: W rows, then tokens
  static constexpr int kPerWave = (kChunks + 3) / 4;    // copies per copying wavefront per stage
  static constexpr int kStageBytes = kChunks * 1024;
  static constexpr int kSteps = 2;                      // stages per barrier
  static constexpr int kDepth = 8;                      // stages in the ring
  static constexpr int kScratch = kDepth * kStageBytes; // 1 KB target of padding copies
  static constexpr int kScales = kScratch + 1024;       // scale chunks: block b, chunk c at (b kChunks + c) KB
};
// LDS bytes of the balanced MXFP4 decode kernel for G groups and K (0 if K does not fit).
template <int G>
int mx_dw_lds_bytes_g(int64_t K) {
  using C = MxDwCfg<G>;
  const int64_t blocks = (K / 256 + 15) / 16;
  const int64_t bytes = C::kScales + blocks * C::kChunks * 1024;
  return bytes <= 160 * 1024 ? (int)bytes : 0;
}

// s_waitcnt for at most n stages of P copies each still in flight (n <= 4).
template <int P>
__device__ __forceinline__ void mx_dw_wait_stages(int n) {
  static_assert(4 * P <= 63, "wait cases");
  switch (n) {
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * P)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * P)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * P)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1 * P)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
  }
}

template <int G>
__global__ __launch_bounds__(kDwThreads) void gemm_mx_decode_rows_kernel(GemmArgs g, int rows_per_wg) {
  using C = MxDwCfg<G>;
  constexpr int S = C::kSteps, D = C::kDepth, NA = (G + 1) / 2;
  static_assert(D - 2 * S <= 4, "wait cases");
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r0 = blockIdx.x * rows_per_wg;
  const int rw = min(rows_per_wg, g.N - r0);             // rows of this workgroup (>= 1)
  const uint32_t kb = (uint32_t)g.K / 2, kx = (uint32_t)g.K / 32;
  const int nst = g.K / 256;
  const uint8_t* wcb = g.w_codes + (size_t)r0 * kb;
  const uint8_t* wxb = g.w_scales + (size_t)r0 * kx;

  // Row of the stage's row list that lane l copies in chunk c: W row min(8c + l/8, rw - 1) of
  // the workgroup, or token row min(8(c - 4G) + l/8, M - 1); chunks past the list copy row 0.
  auto list_row = [&](int c, uint32_t pitch) -> uint32_t {
    const int i = lane >> 3;
    if (c < 4 * G) return (uint32_t)min(8 * c + i, rw - 1) * pitch;
    if (c < C::kChunks) return (uint32_t)min(8 * (c - 4 * G) + i, g.M - 1) * pitch;
    return 0u;
  };
  const bool copier = wave < 4;
  uint32_t row_off[C::kPerWave];
#pragma unroll
  for (int i = 0; i < C::kPerWave; ++i) row_off[i] = list_row((wave & 3) + 4 * i, kb);
  // Lane l copies 16 B piece (l & 7) ^ (l >> 3) of row l >> 3 into slot l & 7 of that row.
  const uint32_t piece16 = (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  auto copy_codes = [&](int t) {
    uint8_t* stage = lds + (t % D) * C::kStageBytes;
#pragma unroll
    for (int i = 0; i < C::kPerWave; ++i) {
      const int c = (wave & 3) + 4 * i;
      if (c < C::kChunks)
        copy16_to_lds(c < 4 * G ? wcb : g.a_codes, row_off[i] + piece16 + (uint32_t)t * 128, stage + c * 1024);
      else
        copy16_to_lds(wcb, row_off[i] + piece16 + (uint32_t)t * 128, lds + C::kScratch);
    }
  };

  // Scale bytes, all stages: block b (stages 16b .. 16b+15), chunk c = rows 8c .. 8c+7, piece q
  // of a row = stages 16b + 2q and 16b + 2q + 1; pieces past the last stage repeat the last pair.
  {
    const int nblk = (nst + 15) / 16;
    const int q = (lane & 7) ^ (lane >> 3);
    for (int e = wave; e < nblk * C::kChunks; e += 8) {
      const int b = e / C::kChunks, c = e - b * C::kChunks;
      const uint32_t off = list_row(c, kx) + (uint32_t)min(16 * b + 2 * q, nst - 2) * 8;
      copy16_to_lds(c < 4 * G ? wxb : g.a_scales, off, lds + C::kScales + e * 1024);
    }
  }
  if (copier) {
    for (int t = 0; t < D - S && t < nst; ++t) copy_codes(t);
  } else {
    // The loop's waits count stage copies, which these wavefronts do not issue: their scale
    // copies must be complete before the first barrier.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }

  const int r = lane & 31, h = lane >> 5, piece = wave & 3, iw = r & 7;
  const int tok = 4 * G + ((r & 15) >> 3);                // token chunk of this lane
  const int code_slot = dl_slot(iw, 2 * piece + h);
  const uint32_t ssh = 8u * (uint32_t)((2 * piece + h) & 3);
  f32x16_t acc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) acc[i] = f32x16_t{};

  for (int t0 = 0; t0 < nst; t0 += S) {
    // Stages t0 .. t0+S-1 must be complete; copies issued after them (up to stage
    // t0 + D - S - 1, at most D - 2S stages) may still be in flight.
    mx_dw_wait_stages<C::kPerWave>(min(t0 + D - S - 1, nst - 1) - min(t0 + S - 1, nst - 1));
    asm volatile("" ::: "memory");
    __syncthreads();            // this step's stages copied by every wavefront; the last step's read by all
    if (copier) {
#pragma unroll
      for (int u = 0; u < S; ++u)
        if (t0 + D - S + u < nst) copy_codes(t0 + D - S + u);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int t = t0 + u;
      if (t < nst) {
        const uint8_t* stage = lds + (t % D) * C::kStageBytes;
        const uint8_t* sc = lds + C::kScales + (t >> 4) * C::kChunks * 1024;
        const int sp = dl_slot(iw, (t & 15) >> 1) + 8 * (t & 1) + 4 * (piece >> 1);
        const uint4 a = *reinterpret_cast<const uint4*>(stage + tok * 1024 + code_slot);
        const uint32_t as = *reinterpret_cast<const uint32_t*>(sc + tok * 1024 + sp) >> ssh;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          const int j = (wave >> 2) + 2 * i;              // W group
          if (j < G) {
            const int wc = 4 * j + (r >> 3);
            const uint4 w = *reinterpret_cast<const uint4*>(stage + wc * 1024 + code_slot);
            const uint32_t ws = *reinterpret_cast<const uint32_t*>(sc + wc * 1024 + sp) >> ssh;
            acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp4_operand(a), fp4_operand(w), acc[i], 4, 4,
                                                                     0, (int)as, 0, (int)ws);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Sum the four wavefronts of each group in a fixed order, then scale and store.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  __syncthreads();              // every wavefront is done with the ring
  f32x16_t* red = reinterpret_cast<f32x16_t*>(lds);
#pragma unroll
  for (int i = 0; i < NA; ++i) red[(wave * NA + i) * 64 + lane] = acc[i];
  __syncthreads();
  if (wave < G) {
    const int j = wave, half = j & 1, i = j >> 1;
    f32x16_t sum = red[((4 * half) * NA + i) * 64 + lane];
    for (int p = 1; p < 4; ++p) sum += red[((4 * half + p) * NA + i) * 64 + lane];
    const int nl = 32 * j + r, n = r0 + nl;
    if (nl < rw) {
      const float sw = w_global_at(g, n);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int m = 8 * (q >> 2) + 4 * h + (q & 3);
        if (m < g.M) store_out(g, m, n, (sum[q] * g.a_global[g.a_per_row ? m : 0]) * sw);
      }
    }
  }
}

// ------------------------------------------------------------------ decode, one or two tokens

// One token (batch-1 decode), K a multiple of 64, Y in fp32 or bf16: a matrix-vector product on
// the vector ALUs instead of MFMA.  The MFMA decode kernels pad the token to 16 rows and the W
// rows to 16-row groups and dequantize both operands in every workgroup (about 2.4 VALU
// instructions per useful W value at the MLP down projection, 20 rows per CU); here a W value
// costs half a converter instruction and half a dot2, and its block scale is applied once per 16
// values:
//   p_b  = sum over the block's 16 k of (E2M1(w_k) 2^8) t_k      (v_dot2_f32_f16, fp32)
//   acc += p_b (E4M3(s_b) 2^-8)                                  (one fma per block)
// with t_k = E2M1 E4M3 of the token, exact in fp16, dequantized once per workgroup into LDS.
// Every product is exact in fp32 (11-bit significands).  The roundings -- at most two per dot2
// inside a block's partial, one per block into the lane's sum, seven in the wave's reduction and
// sixteen in the sum over the workgroup's wavefronts -- keep the error well inside 1e-4 sum |a w|.
//
// Workgroup b owns W rows [b R, b R + R), cut into items of 1 KB of codes (2048 values of a row,
// the last item of a row shorter) and their 128 scale bytes; the R x (items per row) items are
// shared out as 16 contiguous, equal ranges, one per wavefront, so every wavefront does the same
// work whatever R is (a range may start and end inside a row).  Lane l multiplies the 16 bytes
// at 16 l (32 values, two blocks) with scale bytes 2 l and 2 l + 1.  Items are copied straight
// into a ring of kGvDepth slots private to the wavefront (one 1 KB copy for the codes, one 256 B
// copy for the scales, lanes 32-63 repeating lanes 0-31), waited for with exact counts (which
// rest on the wavefront's loads completing in issue order, 16-byte and 4-byte copies alike) so
// that kGvDepth - 1 items stay in flight across rows, and read from LDS one item ahead of the
// products; copies past the range re-read its last item, unused.  The token's bytes are copied
// into LDS the same way, before the ring's first copies, so those stay in flight while the token
// is dequantized.  With 16 wavefronts per CU the latency of one wavefront's LDS reads and
// dependent dot2 chain hides behind the others.  The token values sit in LDS zero-padded to whole
// items (codes past a row's end multiply zeros), laid out so that one item's reads of them are
// four 1 KB runs of consecutive LDS from one per-lane base.  A wavefront's sum over its part of a row is reduced
// across its lanes in a fixed order and left in LDS in that row's slot for the wavefront (slots
// of wavefronts that do not touch the row stay zero); the workgroup adds each row's 16 slots in
// order and stores the result.
constexpr int kGvThreads = 1024;
constexpr int kGvWaves = kGvThreads / 64;
constexpr int kGvDepth = 4;
constexpr int kGvSlot = 1024 + 256;                       // codes, then scale bytes (x2)
constexpr int kGvMaxLds = 160 * 1024;

// Sum of v over the wavefront's 64 lanes in a fixed order, without LDS: within each row of 16
// lanes, four DPP exchanges (neighbour in the pair, pair in the quad, quad in the half-row via
// the half-row mirror, half in the row via the row mirror) leave every lane of the row holding
// the same row sum; the four row sums are then read out and added pairwise.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// LDS layout: the token's values (whole items); the token's raw bytes: its codes (whole 1 KB
// copies) and scale bytes (whole 256 B copies), or with the quantization fused in its bf16 values
// (whole 1 KB copies); the rings; the row slots; with the quantization fused, one word per
// wavefront for the row maximum.
struct GvLayout {
  int64_t raw_codes, raw_scales, rings, slots, red, bytes;
  __host__ __device__ GvLayout(int64_t K, int64_t rows, bool quant) {
    const int64_t items = (K + 2047) / 2048;
    raw_codes = items * 4096;
    raw_scales = raw_codes + (quant ? (2 * K + 1023) / 1024 * 1024 : (K / 2 + 1023) / 1024 * 1024);
    rings = raw_scales + (quant ? 0 : (K / 16 + 255) / 256 * 256);
    slots = rings + (int64_t)kGvWaves * kGvDepth * kGvSlot;
    red = slots + rows * kGvWaves * 4;
    bytes = red + (quant ? kGvWaves * 4 : 0);
  }
};

// The token as one bf16 row, quantized inside the kernel (every workgroup computes the same
// bytes; workgroup 0 writes them out): codes [K/2], scale bytes [K/16] and the global scale, which
// is read instead of computed when `given` is set.
struct GvQuant {
  const uint8_t* x;
  uint8_t* codes;
  uint8_t* scales;
  float* global;
  int32_t given;
};
constexpr int kGvQuantBlocks = 2;   // 16-value blocks per thread: K up to 2 * 1024 * 16

template <bool Q>
__global__ __launch_bounds__(kGvThreads) void gemm_gemv_kernel(GemmArgs g, int rows_per_wg, GvQuant q) {
  constexpr int D = kGvDepth;
  static_assert(D % 2 == 0, "the unrolled steps alternate two operand sets");
  extern __shared__ __align__(16) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const uint32_t groups = (uint32_t)g.K / 32, kb = (uint32_t)g.K / 2, ks = (uint32_t)g.K / 16;
  const int nch = (int)((groups + 63) / 64);            // items per row
  const int r0 = blockIdx.x * rows_per_wg;
  const int rows = min(r0 + rows_per_wg, g.N) - r0;
  const GvLayout lay(g.K, rows, Q);
  uint8_t* ring = lds + lay.rings + wave * (D * kGvSlot);
  float* slots = reinterpret_cast<float*>(lds + lay.slots);   // [row][wave]

  const int total = rows * nch;                         // item j = item j % nch of row j / nch
  const int it0 = wave * total / kGvWaves, it1 = (wave + 1) * total / kGvWaves;
  const int items = it1 - it0;

  // The token's bytes into LDS: copy c (codes 1 KB at a time, then scale bytes 256 B at a time;
  // with the quantization fused, bf16 values 1 KB at a time; lanes past the end re-reading the
  // last piece into the padding) is wavefront c % 16's.
  if constexpr (Q) {
    const uint32_t xb = 2u * (uint32_t)g.K;
    for (int c = wave; c < (int)((xb + 1023) / 1024); c += kGvWaves)
      copy16_to_lds(q.x, min(1024u * c + 16u * lane, xb - 16u), lds + lay.raw_codes + 1024 * c);
  } else {
    const int ncode = (int)((kb + 1023) / 1024), nscale = (int)((ks + 255) / 256);
    for (int c = wave; c < ncode + nscale; c += kGvWaves) {
      if (c < ncode)
        copy16_to_lds(g.a_codes, min(1024u * c + 16u * lane, kb - 16u), lds + lay.raw_codes + 1024 * c);
      else
        copy4_to_lds(g.a_scales, min(256u * (c - ncode) + 4u * lane, ks - 4u), lds + lay.raw_scales + 256 * (c - ncode));
    }
  }

  // Ring copies: the wavefront's items in order, item t into slot t % D; past it1 - 1 the last
  // item again.  The copy position advances through W's rows by pointer (rows are contiguous).
  const int r_first = it0 / nch;
  int cc = it0 - r_first * nch, j_copy = it0;
  const uint8_t* cp_codes = g.w_codes + (size_t)(r0 + r_first) * kb;
  const uint8_t* cp_scales = g.w_scales + (size_t)(r0 + r_first) * ks;
  const uint32_t lane16 = 16u * (uint32_t)lane, lane4 = 4u * (uint32_t)(lane & 31);
  auto copy_next = [&](int u) {
    copy16_to_lds(cp_codes, min(lane16 + 1024u * (uint32_t)cc, kb - 16u), ring + u * kGvSlot);
    copy4_to_lds(cp_scales, min(lane4 + 128u * (uint32_t)cc, ks - 4u), ring + u * kGvSlot + 1024);
    if (j_copy + 1 < it1) {
      ++j_copy;
      if (++cc == nch) {
        cc = 0;
        cp_codes += kb;
        cp_scales += ks;
      }
    }
  };
  if (items > 0) {
#pragma unroll
    for (int u = 0; u < D; ++u) copy_next(u);
  }

  // The row slots start at zero.
  for (int t = threadIdx.x; t < rows * kGvWaves; t += kGvThreads) slots[t] = 0.0f;
  // This wavefront's token copies are older than its 2 D ring copies (none if it has no items:
  // then the wait is for all of them).
  if (items > 0)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * D));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  __syncthreads();
  // The token's values, E2M1 * E4M3 in fp16 (exact), zeros past K.  32-value group s = 64 c + l
  // sits as four 16 B pieces at c 4096 + q 1024 + 16 l (q = 0..3), so that a wavefront reading
  // piece q of groups 64 c .. 64 c + 63 reads 1 KB of consecutive LDS.
  float a_g;                                            // the token's global scale
  if constexpr (Q) {
    // Quantize the bf16 row as the quantizer's per-row mode does: s_g = fl32(max |x| / 2688)
    // from the integer max of the magnitude bits (NaN propagates), or the given scale, then
    // encode_block per 16 values.  Block b = 16 values = pieces 2 (b & 1), 2 (b & 1) + 1 of
    // group b >> 1.
    const uint32_t bpr = (uint32_t)g.K / 16, bpad = (uint32_t)nch * 128;
    float v[kGvQuantBlocks][16];
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < kGvQuantBlocks; ++j) {
      const uint32_t b = threadIdx.x + j * kGvThreads;
      if (b < bpr) {
        const uint4 w0 = *reinterpret_cast<const uint4*>(lds + lay.raw_codes + 32 * b);
        const uint4 w1 = *reinterpret_cast<const uint4*>(lds + lay.raw_codes + 32 * b + 16);
        widen(w0, v[j], (const uint16_t*)nullptr);
        widen(w1, v[j] + 8, (const uint16_t*)nullptr);
        m = max(m, max(max_abs_bits(w0, (const uint16_t*)nullptr), max_abs_bits(w1, (const uint16_t*)nullptr)));
      }
    }
    if (q.given) {
      // A scalar load waited for in the same statement: a vector load here would be counted
      // with the ring's copies, and waiting for it would drain them.
      uint32_t bits;
      asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(bits) : "s"(q.global) : "memory");
      a_g = __uint_as_float(bits);
    } else {
      uint32_t* red = reinterpret_cast<uint32_t*>(lds + lay.red);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
      if (lane == 0) red[wave] = m;
      __syncthreads();
      m = red[0];
#pragma unroll
      for (int w = 1; w < kGvWaves; ++w) m = max(m, red[w]);
      a_g = __uint_as_float(m) / kGlobalDivisor;
      if (blockIdx.x == 0 && threadIdx.x == 0) q.global[0] = a_g;
    }
#pragma unroll
    for (int j = 0; j < kGvQuantBlocks; ++j) {
      const uint32_t b = threadIdx.x + j * kGvThreads;
      if (b < bpad) {
        half8_t lo8 = half8_t{}, hi8 = half8_t{};
        if (b < bpr) {
          uint32_t sb, lo, hi;
          encode_block(v[j], a_g, sb, lo, hi);
          if (blockIdx.x == 0) {
            *reinterpret_cast<uint2*>(q.codes + 8 * (size_t)b) = make_uint2(lo, hi);
            q.scales[b] = (uint8_t)sb;
          }
          const half2_t sp = scale_pair_f16(sb);
          lo8 = dequant8_f16(lo, sp);
          hi8 = dequant8_f16(hi, sp);
        }
        const uint32_t gs = b >> 1;
        uint8_t* dst = lds + (gs >> 6) * 4096 + 2048 * (b & 1) + 16 * (gs & 63);
        *reinterpret_cast<half8_t*>(dst) = lo8;
        *reinterpret_cast<half8_t*>(dst + 1024) = hi8;
      }
    }
  } else {
    for (uint32_t s = threadIdx.x; s < (uint32_t)nch * 64; s += kGvThreads) {
      half8_t v[4] = {half8_t{}, half8_t{}, half8_t{}, half8_t{}};
      if (s < groups) {
        const uint4 c = *reinterpret_cast<const uint4*>(lds + lay.raw_codes + 16 * s);
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(lds + lay.raw_scales + 2 * s);
        const half2_t p0 = scale_pair_f16(sc & 0xFFu), p1 = scale_pair_f16(sc >> 8);
        v[0] = dequant8_f16(c.x, p0);
        v[1] = dequant8_f16(c.y, p0);
        v[2] = dequant8_f16(c.z, p1);
        v[3] = dequant8_f16(c.w, p1);
      }
      uint8_t* dst = lds + (s >> 6) * 4096 + 16 * (s & 63);
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<half8_t*>(dst + 1024 * j) = v[j];
    }
    a_g = 0.0f;
  }
  // The W pointers' scalar loads must not stay pending into the loop, where their first use
  // would wait for every LDS read as well: the empty statement takes them in scalar registers
  // here, and the wait (LDS and scalar loads only) completes them.
  asm volatile("" : : "s"(g.w_codes), "s"(g.w_scales));
  __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0)
  __syncthreads();

  // Item i is read from LDS one item ahead: its codes, scale bytes and token values are in
  // registers while item i - 1 is multiplied, so the LDS latency hides behind that work.  The
  // loop is unrolled D times, so ring slots are fixed offsets and the two operand sets
  // alternate without copies.
  struct Operands {
    uint4 wq;
    uint32_t sc;
    half8_t t[4];
  };
  auto read_item = [&](int u, int c, Operands& o) {
    const uint8_t* slot = ring + u * kGvSlot;
    o.wq = *reinterpret_cast<const uint4*>(slot + lane16);
    o.sc = *reinterpret_cast<const uint16_t*>(slot + 1024 + 2 * lane);
    const uint8_t* tok = lds + c * 4096 + lane16;
#pragma unroll
    for (int q = 0; q < 4; ++q) o.t[q] = *reinterpret_cast<const half8_t*>(tok + 1024 * q);
  };
  float acc = 0.0f;
  int jr = r_first, jc = it0 - r_first * nch;
  Operands op[2];
  // Item 0's two copies are older than the 2 (D - 1) of the items after it.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (D - 1)));
  asm volatile("" ::: "memory");
  read_item(0, jc, op[0]);
  for (int i0 = 0; i0 < items; i0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (i0 + u < items) {
        Operands& cur = op[u & 1];
        // Item i + 1 (past the last one: a slot of unused copies, read and dropped).
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * (D - 2)));
        asm volatile("" ::: "memory");
        read_item((u + 1) % D, jc + 1 == nch ? 0 : jc + 1, op[(u + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          float p = 0.0f;
#pragma unroll
          for (int q = 2 * b; q < 2 * b + 2; ++q) {
            const uint32_t wd = q == 0 ? cur.wq.x : q == 1 ? cur.wq.y : q == 2 ? cur.wq.z : cur.wq.w;
            const half2_t h[4] = {__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 256.0f, 0),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 256.0f, 1),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 256.0f, 2),
                                  __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd, 256.0f, 3)};
#pragma unroll
            for (int k = 0; k < 4; ++k)
              p = __builtin_amdgcn_fdot2(h[k], half2_t{cur.t[q][2 * k], cur.t[q][2 * k + 1]}, p, false);
          }
          acc = __builtin_fmaf(p, (float)scale_pair_f16((cur.sc >> (8 * b)) & 0xFFu)[0], acc);
        }
        __builtin_amdgcn_sched_barrier(0);
        // The refill below overwrites the slot that item i was read from.  Those reads must be
        // complete first; the sum above consumes every value they loaded, so taking it as an
        // operand here places the copy after the compiler's own wait for them (without it the
        // compiler may issue the copy ahead of that wait and of the arithmetic).
        asm volatile("" : : "v"(acc) : "memory");
        copy_next(u);                                    // item i's slot, for item i + D
        if (jc + 1 == nch || i0 + u + 1 == items) {      // end of this wavefront's part of row jr
          const float v = wave_sum_dpp(acc);
          if (lane == 0) slots[jr * kGvWaves + wave] = v;
          acc = 0.0f;
        }
        if (++jc == nch) {
          jc = 0;
          ++jr;
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));             // copies past the last item
  asm volatile("" ::: "memory");
  __syncthreads();
  for (int t = threadIdx.x; t < rows; t += kGvThreads) {
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < kGvWaves; ++w) v += slots[t * kGvWaves + w];
    store_out(g, 0, r0 + t, (v * (Q ? a_g : g.a_global[0])) * w_global_at(g, r0 + t));
  }
}

// ------------------------------------------------------------------ plain kernel

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float v = mag[c & 7u];
  return (c & 8u) ? -v : v;
}

__global__ __launch_bounds__(256) void gemm_plain_kernel(GemmArgs g) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)g.M * g.N) return;
  const int m = (int)(idx / g.N), n = (int)(idx % g.N);
  const int64_t kb = g.K / 2, ks = g.K / 16;
  float acc = 0.0f;
  for (int b = 0; b < g.K / 16; ++b) {
    const float sa = e4m3_decode(g.a_scales[m * ks + b]);
    const float sw = e4m3_decode(g.w_scales[n * ks + b]);
    for (int i = 0; i < 8; ++i) {
      const uint32_t ca = g.a_codes[m * kb + b * 8 + i], cw = g.w_codes[n * kb + b * 8 + i];
      acc = __builtin_fmaf(e2m1_value(ca & 15u) * sa, e2m1_value(cw & 15u) * sw, acc);
      acc = __builtin_fmaf(e2m1_value(ca >> 4) * sa, e2m1_value(cw >> 4) * sw, acc);
    }
  }
  const float v = (acc * g.a_global[g.a_per_row ? m : 0]) * w_global_at(g, n);
  store_out(g, m, n, v);
  if (g.gate_h > 0 && n >= g.gate_n0) store_gate(g, m, n, v);
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  (void)M;
  (void)N;
  (void)K;
  return 0;   // no path needs device scratch
}

namespace {

GemmArgs gemm_args(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                   const float* a_global, int a_global_per_row, const uint8_t* w_codes, const uint8_t* w_scales,
                   const float* w_globals, const SegmentTable& seg, void* y, int y_dtype, int64_t ldy) {
  GemmArgs g;
  g.M = (int32_t)M;
  g.N = (int32_t)N;
  g.K = (int32_t)K;
  g.a_codes = a_codes;
  g.a_scales = a_scales;
  g.a_global = a_global;
  g.a_per_row = a_global_per_row;
  g.w_codes = w_codes;
  g.w_scales = w_scales;
  g.w_globals = w_globals;
  g.y = y;
  g.y_bf16 = y_dtype == NVFP4_BF16;
  g.ldy = ldy;
  g.y_vec = reinterpret_cast<uintptr_t>(y) % 16 == 0 && (ldy * (g.y_bf16 ? 2 : 4)) % 16 == 0;
  g.seg = seg;
  g.q_out = 0;
  g.q_global = nullptr;
  g.q_codes = nullptr;
  g.q_scales = nullptr;
  g.gate_n0 = (int32_t)N;
  g.gate_h = 0;
  g.gate_a_log = nullptr;
  g.gate_dt_bias = nullptr;
  g.gate_g = nullptr;
  g.gate_beta = nullptr;
  g.swiglu = 0;
  return g;
}

// Rows per workgroup of the balanced decode kernel: the fewest rounds over the CUs with at
// most cap rows per workgroup (the largest multiple of unit up to 16 kDwMaxG), the rows then
// spread evenly over the workgroups of those rounds and rounded up to a multiple of unit (16
// for NVFP4 output, whose 16-column blocks must not straddle workgroups; 32 for SwiGLU pairs;
// else 1); that stays within cap, as N <= rounds * CUs * cap.  SwiGLU pairs may take three per
// workgroup (96 rows) where K leaves room in LDS: with two, the rounding to whole pairs adds a
// short last round, and a workgroup's time is mostly its K loop's latency, not its rows.
// Returns the kernel's LDS bytes, 0 when K is too long for its LDS.
int decode_rows_plan(int64_t N, int64_t K, int cus, int unit, int& rows, int& groups) {
  const int64_t cap = unit == 32 && dw_lds_bytes(kDwPairG, K) ? 16 * kDwPairG : 16 * kDwMaxG / unit * unit;
  const int64_t rounds = (N + cus * cap - 1) / (cus * cap);
  int64_t r = (N + cus * rounds - 1) / (cus * rounds);
  r = (r + unit - 1) / unit * unit;
  rows = (int)r;
  groups = (int)((r + 15) / 16);
  return dw_lds_bytes(groups, K);
}

template <int G>
int set_decode_rows_lds() {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_decode_rows_kernel<G, false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_decode_rows_kernel<G, true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
}

// Rows per workgroup of the balanced MXFP4 decode kernel: the fewest rounds over the CUs with at
// most 96 rows per workgroup (64 where K leaves no room for three groups in LDS), the rows then
// spread evenly over the workgroups of those rounds.  Returns the kernel's LDS bytes, 0 when it
// does not apply (one group is enough, or K does not fit).
int mx_decode_rows_plan(int64_t N, int64_t K, int cus, int& rows, int& groups) {
  const int64_t cap = mx_dw_lds_bytes_g<3>(K) ? 96 : 64;
  const int64_t rounds = (N + cus * cap - 1) / (cus * cap);
  const int64_t r = (N + cus * rounds - 1) / (cus * rounds);
  rows = (int)r;
  groups = (int)((r + 31) / 32);
  return groups == 3 ? mx_dw_lds_bytes_g<3>(K) : groups == 2 ? mx_dw_lds_bytes_g<2>(K) : 0;
}

template <int G>
void launch_decode_rows(const GemmArgs& g, bool gated, int rows, int lds_bytes, hipStream_t stream) {
  const unsigned grid = (unsigned)((g.N + rows - 1) / rows);
  if (gated)
    gemm_decode_rows_kernel<G, true><<<grid, kDwThreads, lds_bytes, stream>>>(g, rows);
  else
    gemm_decode_rows_kernel<G, false><<<grid, kDwThreads, lds_bytes, stream>>>(g, rows);
}

// One 256 x 256 tile per CU at a time.  If the last round of tiles would fill at most half of
// the CUs, enough whole tile columns move to 128 x 128 tiles to absorb it: workgroups
// [0, big) take 256 x 256 tiles of columns [0, n_split), the other `small` 128 x 128 tiles.
void tile_grid(int64_t M, int64_t N, int cus, int64_t& n_split, int64_t& big, int64_t& small) {
  const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
  const int64_t rem = (tm * tn) % cus;
  int64_t peel = 0;
  n_split = N;
  if (rem > 0 && rem <= cus / 2) {
    peel = (rem + tm - 1) / tm;
    if (peel >= tn) peel = 0;
    n_split = (tn - peel) * 256;
  }
  big = tm * ((n_split + 255) / 256);
  small = peel ? ((M + 127) / 128) * ((N - n_split + 127) / 128) : 0;
}

}  // namespace

// Once per device (device.hip), with the device current: raise the dynamic LDS limit of every
// kernel whose LDS exceeds the default.
int gemm_device_setup() {
  const void* tiles[] = {reinterpret_cast<const void*>(gemm_prefill_kernel<kEpiStore>),
                         reinterpret_cast<const void*>(gemm_prefill_kernel<kEpiNvfp4>),
                         reinterpret_cast<const void*>(gemm_prefill_kernel<kEpiGates>),
                         reinterpret_cast<const void*>(gemm_prefill_kernel<kEpiSwiglu>),
                         reinterpret_cast<const void*>(gemm_mx_kernel)};
  for (const void* k : tiles)
    if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kPrefillLds) != hipSuccess)
      return NVFP4_ERR_HIP;
  for (int wc = 2; wc <= 4; ++wc)
    for (int tc = 1; tc <= 2; ++tc)
      for (const DecodeLdsKernel k : {decode_lds_kernel(false, wc, tc), decode_lds_kernel(true, wc, tc),
                                      mx_decode_lds_kernel(wc, tc)})
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                kDlLds) != hipSuccess)
          return NVFP4_ERR_HIP;
  const void* decode[] = {reinterpret_cast<const void*>(gemm_decode_q4_kernel<4, false>),
                          reinterpret_cast<const void*>(gemm_decode_q4_kernel<4, true>),
                          reinterpret_cast<const void*>(gemm_decode_q4_kernel<5, false>),
                          reinterpret_cast<const void*>(gemm_decode_q4_kernel<5, true>)};
  for (const void* k : decode)
    if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kDlLds) != hipSuccess)
      return NVFP4_ERR_HIP;

  if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_gemv_kernel<false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kGvMaxLds) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_gemv_kernel<true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kGvMaxLds) != hipSuccess)
    return NVFP4_ERR_HIP;
  int st = set_decode_rows_lds<1>();
  if (st == NVFP4_OK) st = set_decode_rows_lds<2>();
  if (st == NVFP4_OK) st = set_decode_rows_lds<3>();
  if (st == NVFP4_OK) st = set_decode_rows_lds<4>();
  if (st == NVFP4_OK) st = set_decode_rows_lds<5>();
  if (st == NVFP4_OK) st = set_decode_rows_lds<kDwPairG>();
  if (st != NVFP4_OK) return st;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_mx_decode_rows_kernel<2>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess ||
      hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_mx_decode_rows_kernel<3>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
    return NVFP4_ERR_HIP;
  return NVFP4_OK;
}

int launch_decode_linear(int64_t N, int64_t K, const uint16_t* x, bool given, uint8_t* a_codes, uint8_t* a_scales,
                         float* a_global, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                         void* y, int y_dtype, hipStream_t stream) {
  if (N == 0) return NVFP4_OK;
  if (K % 64 != 0 || (K + 2047) / 2048 * 128 > (int64_t)kGvQuantBlocks * kGvThreads) return NVFP4_ERR_UNSUPPORTED;
  DeviceInfo dev;
  const int st = device_info(stream, dev);
  if (st != NVFP4_OK) return st;
  const int64_t rows = (N + dev.cus - 1) / dev.cus;
  const GvLayout lay(K, rows, true);
  if (lay.bytes > kGvMaxLds) return NVFP4_ERR_UNSUPPORTED;
  SegmentTable seg{};
  seg.count = 1;
  seg.bound[0] = 0;
  seg.bound[1] = (int32_t)N;
  const GemmArgs g = gemm_args(1, N, K, a_codes, a_scales, a_global, 0, w_codes, w_scales, w_global, seg, y,
                               y_dtype, N);
  const GvQuant q{reinterpret_cast<const uint8_t*>(x), a_codes, a_scales, a_global, given ? 1 : 0};
  gemm_gemv_kernel<true><<<(unsigned)((N + rows - 1) / rows), kGvThreads, (size_t)lay.bytes, stream>>>(g, (int)rows, q);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                const float* a_global, int a_global_per_row, const uint8_t* w_codes, const uint8_t* w_scales,
                const float* w_globals, const SegmentTable& seg, void* y, int y_dtype, int64_t ldy, void* workspace,
                hipStream_t stream, const QuantOut* qout, const GateOut* gates, bool swiglu) {
  (void)workspace;
  if (M == 0 || N == 0) return NVFP4_OK;
  // The tiled and decode kernels address a row of W or A with 32-bit per-lane offsets from a
  // per-tile base (row index times the row pitch, up to 96 rows at once; 24-bit multiplies in
  // the prefill tiles): K below 2^24 keeps every such offset in range.  Larger K, and K that
  // is not a multiple of 128 (or of 256 past 16 tokens), take the plain kernel.
  const bool plain = K % 128 != 0 || K >= (1 << 24) || (M > 16 && K % BK != 0);
  if ((qout || swiglu) && (plain || N % 16 != 0)) return NVFP4_ERR_UNSUPPORTED;
  if ((qout || swiglu) && gates) return NVFP4_ERR_INVALID_ARG;
  if (swiglu && N % 32 != 0) return NVFP4_ERR_INVALID_ARG;
  GemmArgs g = gemm_args(M, N, K, a_codes, a_scales, a_global, a_global_per_row, w_codes, w_scales, w_globals, seg,
                         y, y_dtype, ldy);
  g.q_out = qout != nullptr;
  g.q_global = qout ? qout->global : nullptr;
  g.q_codes = qout ? qout->codes : nullptr;
  g.q_scales = qout ? qout->scales : nullptr;
  g.gate_n0 = gates ? gates->n0 : (int32_t)N;
  g.gate_h = gates ? gates->h : 0;
  g.gate_a_log = gates ? gates->a_log : nullptr;
  g.gate_dt_bias = gates ? gates->dt_bias : nullptr;
  g.gate_g = gates ? gates->g : nullptr;
  g.gate_beta = gates ? gates->beta : nullptr;
  g.swiglu = swiglu;
  const bool gated = gates != nullptr;
  int cus_gv = 0;
  if (M == 1 && K % 64 == 0 && !qout && !swiglu && !gated) {
    DeviceInfo dev;
    const int st = device_info(stream, dev);
    if (st != NVFP4_OK) return st;
    cus_gv = dev.cus;
  }
  // Past one round of 32-row workgroups with whole 256-wide stages the balanced MFMA kernel
  // streams W faster than this one; below it the matrix-vector kernel beats the K-split kernel.
  if (cus_gv && N > (int64_t)kDecodeRows * cus_gv && K % 256 == 0) cus_gv = 0;
  const int64_t gv_rows = cus_gv ? (N + cus_gv - 1) / cus_gv : 0;
  if (cus_gv && GvLayout(K, gv_rows, false).bytes <= kGvMaxLds) {
    // Batch-1 decode: one workgroup of about N / CUs rows per CU.
    const unsigned grid = (unsigned)((N + gv_rows - 1) / gv_rows);
    gemm_gemv_kernel<false><<<grid, kGvThreads, (size_t)GvLayout(K, gv_rows, false).bytes, stream>>>(
        g, (int)gv_rows, GvQuant{});
  } else if (plain) {
    const int64_t total = M * N;
    gemm_plain_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(g);
  } else if (M <= 16 && K % 256 == 0) {
    DeviceInfo dev;
    const int st = device_info(stream, dev);
    if (st != NVFP4_OK) return st;
    const int cus = dev.cus;
    // Up to one round of 32-row workgroups the K-split kernel is the faster; past it, the
    // balanced kernel avoids the partial last round.
    int rows = 0, groups = 0;
    const int unit = swiglu ? 32 : g.q_out ? 16 : 1;
    const int lds_bytes = N > (int64_t)kDecodeRows * cus ? decode_rows_plan(N, K, cus, unit, rows, groups) : 0;
    if (lds_bytes == 0) {
      // Rows per workgroup: about N / CUs, so that every CU takes a share (16 to 32; 32 for
      // NVFP4 output, whose 16-column blocks must not straddle workgroups, and for SwiGLU
      // pairs, one pair per workgroup).
      const int64_t share = (N + cus - 1) / cus;
      const int r = unit > 1 ? kDecodeRows : (int)std::min<int64_t>(kDecodeRows, std::max<int64_t>(16, share));
      const unsigned grid = (unsigned)((N + r - 1) / r);
      // Up to 4 tokens and 20 rows (four or five 4-row groups) the 4 x 4 x 4 kernel dequantizes
      // no padding and copies no padding chunk, and is the faster (at the MLP down projection,
      // 5120 x 17408: 12.6-12.9 against 15.6-16.0 us at M = 2-4); past that its instruction
      // rate costs more than the padding it saves.
      if (M <= 4 && r <= 16)
        (gated ? gemm_decode_q4_kernel<4, true> : gemm_decode_q4_kernel<4, false>)<<<grid, kDecodeThreads, kDlLds, stream>>>(g, r);
      else if (M <= 4 && r <= 20)
        (gated ? gemm_decode_q4_kernel<5, true> : gemm_decode_q4_kernel<5, false>)<<<grid, kDecodeThreads, kDlLds, stream>>>(g, r);
      else
        decode_lds_kernel(gated, (r + 7) / 8, M <= 8 ? 1 : 2)<<<grid, kDecodeThreads, kDlLds, stream>>>(g, r);
    } else {
      if (swiglu && groups % 2 != 0) return NVFP4_ERR_UNSUPPORTED;   // not reached: rows % 32 == 0
      switch (groups) {
        case 1: launch_decode_rows<1>(g, gated, rows, lds_bytes, stream); break;
        case 2: launch_decode_rows<2>(g, gated, rows, lds_bytes, stream); break;
        case 3: launch_decode_rows<3>(g, gated, rows, lds_bytes, stream); break;
        case 4: launch_decode_rows<4>(g, gated, rows, lds_bytes, stream); break;
        case 5: launch_decode_rows<5>(g, gated, rows, lds_bytes, stream); break;
        case kDwPairG: launch_decode_rows<kDwPairG>(g, gated, rows, lds_bytes, stream); break;
        default: return NVFP4_ERR_UNSUPPORTED;   // not reached: the plan caps the rows
      }
    }
  } else if (M <= 16) {
    const unsigned grid = (unsigned)((N + kDecodeRows - 1) / kDecodeRows);
    if (gated)
      gemm_decode_kernel<true><<<grid, kDecodeThreads, 0, stream>>>(g);
    else
      gemm_decode_kernel<false><<<grid, kDecodeThreads, 0, stream>>>(g);
  } else {
    DeviceInfo dev;
    const int st = device_info(stream, dev);
    if (st != NVFP4_OK) return st;
    int64_t n_split, big, small;
    tile_grid(M, N, dev.cus, n_split, big, small);
    const unsigned grid = (unsigned)(big + small);
    if (swiglu)
      gemm_prefill_kernel<kEpiSwiglu><<<grid, kPrefillThreads, kPrefillLds, stream>>>(g, (int)n_split, (int)big);
    else if (g.q_out)
      gemm_prefill_kernel<kEpiNvfp4><<<grid, kPrefillThreads, kPrefillLds, stream>>>(g, (int)n_split, (int)big);
    else if (gated)
      gemm_prefill_kernel<kEpiGates><<<grid, kPrefillThreads, kPrefillLds, stream>>>(g, (int)n_split, (int)big);
    else
      gemm_prefill_kernel<kEpiStore><<<grid, kPrefillThreads, kPrefillLds, stream>>>(g, (int)n_split, (int)big);
  }
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                   const float* a_global, int a_global_per_row, const uint8_t* w_codes, const uint8_t* w_scales,
                   const float* w_globals, const SegmentTable& seg, void* y, int y_dtype, int64_t ldy,
                   hipStream_t stream) {
  if (M == 0 || N == 0) return NVFP4_OK;
  if (K % BK != 0 || K >= (1 << 24)) return NVFP4_ERR_UNSUPPORTED;
  const GemmArgs g = gemm_args(M, N, K, a_codes, a_scales, a_global, a_global_per_row, w_codes, w_scales,
                               w_globals, seg, y, y_dtype, ldy);
  if (M <= 16 && K % 512 == 0) {
    DeviceInfo dev;
    const int st = device_info(stream, dev);
    if (st != NVFP4_OK) return st;
    const int cus = dev.cus;
    if (N > 32 * (int64_t)cus) {
      // More rows than one round of 32-row workgroups: the balanced kernel.
      int rows = 0, groups = 0;
      const int lds_bytes = mx_decode_rows_plan(N, K, cus, rows, groups);
      if (lds_bytes > 0) {
        const unsigned grid = (unsigned)((N + rows - 1) / rows);
        if (groups == 3)
          gemm_mx_decode_rows_kernel<3><<<grid, kDwThreads, lds_bytes, stream>>>(g, rows);
        else
          gemm_mx_decode_rows_kernel<2><<<grid, kDwThreads, lds_bytes, stream>>>(g, rows);
        return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
      }
    }
    // Rows per workgroup: the fewest rounds of 32-row workgroups over the CUs, the rows then
    // spread evenly over the workgroups of those rounds (16 to 32 rows), so that no CU takes a
    // whole extra workgroup in a short last round.
    const int64_t rounds = (N + 32 * cus - 1) / (32 * cus);
    const int r = (int)std::min<int64_t>(32, std::max<int64_t>(16, (N + cus * rounds - 1) / (cus * rounds)));
    mx_decode_lds_kernel((r + 7) / 8, M <= 8 ? 1 : 2)<<<(unsigned)((N + r - 1) / r), kDecodeThreads, kDlLds, stream>>>(g, r);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
  }
  if (M <= 16) {
    gemm_mx_decode_kernel<<<(unsigned)((N + kMxDecodeRows - 1) / kMxDecodeRows), kMxDecodeThreads, 0, stream>>>(g);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
  }
  DeviceInfo dev;
  const int st = device_info(stream, dev);
  if (st != NVFP4_OK) return st;
  int64_t n_split, big, small;
  tile_grid(M, N, dev.cus, n_split, big, small);
  gemm_mx_kernel<<<(unsigned)(big + small), kPrefillThreads, kPrefillLds, stream>>>(g, (int)n_split, (int)big);
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4
