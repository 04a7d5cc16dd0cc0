/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 library.
 *
 * The library implements the data-parallel hot path of NVFP4 W4A4 inference of linear
 * layers:
 *   1. activation quantization: per 16-element block a max-abs, an E4M3 block scale under
 *      an FP32 global scale, round-to-nearest-even to E2M1 codes packed two per byte;
 *   2. the block-scaled 4-bit x 4-bit GEMM Y = A . W^T with FP32 accumulation;
 *   3. the fused-module GEMM in which several separately calibrated modules share one
 *      launch and each column segment keeps its own weight global scale (the repair of the
 *      global-scale mismatch);
 *   4. the GEMM whose output leaves already quantized to NVFP4 for the next linear layer;
 *   5. the FP8 (E4M3) key-value cache codec with calibrated per-tensor scales;
 *   6. the fused Gated DeltaNet input projection whose two gate segments leave as the
 *      write strength and the log-space decay, in the same launch;
 *   7. a lossy variant: NVFP4 re-encoded to MXFP4 and multiplied with gfx950's native scaled
 *      FP4 matrix instructions;
 *   8. the gated MLP input projection: the fused gate+up GEMM with its SwiGLU activation in
 *      the same launch, the result optionally leaving as NVFP4 for the down projection;
 *   9. batch-1 decode of one linear layer in one launch: 1 and 2 with the token's quantization
 *      inside the GEMM kernel.
 *
 * Sources: the element format (E2M1 values, one E4M3 scale per 16-element block) is from
 * "NVFP4 W4A4 Quantization Compresses 27B Hybrid Models" (thevalue.engineering), section
 * "Challenging the Recurrence Fragility Assumption"; W4A4 on every linear layer and the
 * 16-element block from "Why Gated DeltaNet Survives 4-Bit Quantization" (kipquest),
 * "The deep dive"; the global-scale mismatch (modules calibrated one by one, run as one
 * fused GEMM under a single scale) and its repair from the paper's abstract (Lattice and
 * kipquest pages).  Each declaration below names the passage its operation follows.
 *
 * Data format (identical for activations and weights):
 *   codes [rows, cols/2]  uint8, row-major, contiguous; two 4-bit E2M1 codes per byte, the
 *                         even column in the low nibble.  Code = sign<<3 | magnitude index,
 *                         magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 *   scales [rows, cols/16] uint8, row-major, contiguous; OCP E4M3FN bytes (bias 7,
 *                         max 448, never NaN), one per 16 consecutive elements of a row.
 *   global scale          float32 on the device: one per tensor, or one per row.
 *   value = E2M1(code) * E4M3(scale) * global_scale.
 *   The dynamic global scale is s_g = fl32(max|x| / 2688), 2688 = 6 * 448.
 *
 * Conventions of every entry point:
 *   * Pointers are DEVICE pointers unless marked (host).  The caller owns all memory; the
 *     library never allocates device memory and never synchronises.  Its only state is set up
 *     once per device by the first call that launches work there (kernel limits, the compute-
 *     unit count, the address of nvfp4_quantize_no_alloc's static array), under std::call_once,
 *     for the device the call's stream belongs to: first calls from several host threads at
 *     once are safe.
 *   * Work is enqueued on `stream` (a hipStream_t passed as void*; NULL = default stream)
 *     and is stream-ordered; the global scales never travel to the host.
 *   * Return value: an nvfp4_status.  Argument errors are detected on the host before any
 *     launch and leave every output untouched.  A failed launch returns NVFP4_ERR_HIP.
 *   * Non-finite input is reported in band: the affected global scale (of the tensor, or of
 *     the row in per-row mode) becomes NaN or infinite and the codes and scales it governs
 *     are unspecified.
 *   * Calls on different streams may run concurrently if their outputs and workspaces do
 *     not overlap.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad enum */
  NVFP4_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. too many segments) */
  NVFP4_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_size */
  NVFP4_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;

typedef enum {
  NVFP4_SCALE_PER_TENSOR = 0, /* s_g = max|x| over the tensor / 2688, written to [1]    */
  NVFP4_SCALE_PER_ROW = 1,    /* s_g[r] = max|x[r,:]| / 2688, written to [rows]         */
  NVFP4_SCALE_GIVEN = 2       /* s_g read from global_scale[0] (a calibrated scale)     */
} nvfp4_scale_mode;

#define NVFP4_MAX_SEGMENTS 64

/*
 * Quantize X[rows, cols] to NVFP4 (format above).  The element format -- E2M1 values with one
 * E4M3 scale per 16-element block -- is the one "NVFP4 W4A4 Quantization Compresses 27B Hybrid
 * Models" describes ("Challenging the Recurrence Fragility Assumption"); "Why Gated DeltaNet
 * Survives 4-Bit Quantization" ("The deep dive") quantizes activations this way at every
 * linear layer, the block of sixteen confining an outlier channel's damage to its own block.
 * The pages imply an FP32 per-module global scale (the mismatch in the paper abstract) without
 * its formula: s_g = fl32(max|x| / 2688) is this library's reading.
 *   x             [rows, ldx] of x_dtype (NVFP4_BF16 or NVFP4_F32); 16-byte aligned, and
 *                 ldx * element size a multiple of 16 bytes; ldx >= cols.
 *   rows >= 0     rows == 0 is a no-op except that PER_TENSOR writes s_g = 0.
 *   cols > 0      multiple of 16.
 *   codes         out [rows, cols/2], 8-byte aligned.
 *   scales        out [rows, cols/16].
 *   global_scale  PER_TENSOR: out [1]; PER_ROW: out [rows]; GIVEN: in [1].  A given scale
 *                 must be finite and > 0 (otherwise the output is unspecified); a zero
 *                 scale (all-zero input) gives all-zero scale bytes and sign-only codes.
 *   workspace     device scratch of nvfp4_quantize_workspace_size() bytes (may be NULL if
 *                 that is 0); contents need no initialisation and are clobbered.
 * Follows: block max -> E4M3 scale -> E2M1 round-to-nearest-even, two codes per byte.
 */
int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                   uint8_t* codes, uint8_t* scales, float* global_scale, int mode,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace nvfp4_quantize needs for this shape and mode (4 KB per tensor, 0
 * per row or given); 0 for a bad shape. */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols, int mode);

/*
 * nvfp4_quantize for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * nvfp4_quantize, without the workspace: the per-tensor mode's partial maxima go to a static
 * device array of the library (4 KB per GPU, held until the process ends) instead.  Allocates
 * nothing, on the host or the device.
 *   Every call on one GPU shares that GPU's array, so calls that overlap in time on one GPU
 *   (different streams, or threads without ordering) race and may return wrong results;
 *   serialise them.  Calls on one stream are ordered and safe.
 *   A shape whose workspace need exceeds the array returns NVFP4_ERR_WORKSPACE (no shape
 *   does at present: the need is at most 4 KB).
 */
int nvfp4_quantize_no_alloc(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t* codes, uint8_t* scales, float* global_scale, int mode, void* stream);

/*
 * The W4A4 linear layer: weights and activations both in the 4-bit block format, as "Why Gated
 * DeltaNet Survives 4-Bit Quantization" ("The deep dive") runs every linear layer of the hybrid
 * model; the paper abstract credits this recipe with the fastest prefill of those compared.
 * Y[M, N] = A . W^T with A = NVFP4 [M, K] activations and W = NVFP4 [N, K] weights, both
 * K-major; FP32 accumulation of the exactly dequantized operands, then
 * y = (acc * a_global[m or 0]) * w_global[0], stored as y_dtype (bf16: round to nearest
 * even).
 *   M >= 0, N >= 0 (zero is a no-op), K > 0 and a multiple of 16.
 *   a_codes, a_scales, w_codes, w_scales 16-byte aligned.
 *   a_global      device [1] (a_global_per_row == 0) or [M] (== 1).
 *   w_global      device [1].
 *   y             [M, ldy] of y_dtype, ldy >= N.
 *   workspace     nvfp4_gemm_workspace_size(M, N, K) bytes (may be NULL if 0; every
 *                 shape needs 0 bytes at present, the argument keeps the ABI stable).
 */
int nvfp4_gemm(int64_t M, int64_t N, int64_t K,
               const uint8_t* a_codes, const uint8_t* a_scales, const float* a_global,
               int a_global_per_row,
               const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
               void* y, int y_dtype, int64_t ldy,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Batch-1 decode of one W4A4 linear layer in one call: the token's activation row is quantized
 * to the 4-bit block format and multiplied with W, as every linear layer of the hybrid model
 * runs at decode ("Why Gated DeltaNet Survives 4-Bit Quantization", "The deep dive": 4-bit
 * weights and activations).  The result is that of
 *   nvfp4_quantize(x, x_dtype, 1, K, K, a_codes, a_scales, a_global, mode, ...)
 *   nvfp4_gemm(1, N, K, a_codes, a_scales, a_global, 0, w_codes, w_scales, w_global, y, y_dtype, N, ...)
 * on the same stream: the token's NVFP4 bytes are written to a_codes / a_scales (and its global
 * scale to a_global, except in NVFP4_SCALE_GIVEN mode, where a_global is read), bit for bit those
 * of nvfp4_quantize, and Y[1, N] to y.  Y is bit for bit that of nvfp4_gemm except where the one
 * launch below runs and nvfp4_gemm takes an MFMA kernel for the shape (bf16 input, K a multiple
 * of 256, N above 32 x the CU count): there both are within nvfp4_gemm's rounding bound of the
 * exact product, accumulated in a different order.
 * With one row NVFP4_SCALE_PER_TENSOR and NVFP4_SCALE_PER_ROW are the same scale; neither needs a
 * workspace here.  For bf16 input with K a multiple of 64 whose working set fits the kernel's
 * 160 KB of LDS (the token twice, as bf16 and as fp16 values, plus the weight copy rings: K up to
 * 18432 for N up to 32512 on 256 CUs) it is one launch that quantizes the token inside the GEMM
 * kernel, with no separate quantize launch; other inputs run the two calls above internally.
 *   N >= 0 (zero: only the quantization), K > 0 and a multiple of 16.
 *   x             device [K] of x_dtype, 16-byte aligned.
 *   a_codes       out [K/2], a_scales out [K/16], both 16-byte aligned; a_global device [1].
 *   w_codes, w_scales, w_global, y_dtype as in nvfp4_gemm; y device [N] of y_dtype.
 */
int nvfp4_decode_linear(int64_t N, int64_t K, const void* x, int x_dtype, int mode,
                        uint8_t* a_codes, uint8_t* a_scales, float* a_global,
                        const uint8_t* w_codes, const uint8_t* w_scales, const float* w_global,
                        void* y, int y_dtype, void* stream);

/*
 * The fused-module GEMM, the repair of the global-scale mismatch the paper abstract reports
 * (modules calibrated one by one, each with its own global scale, served by a kernel that fuses
 * them into one GEMM); "Quantizing All Layers Reveals Recurrent Memory Is Robust" ("Block
 * Scaling and the Geography of Outliers") describes the bug as a single scale applied to every
 * fused module.  W is the concatenation along N of num_segments separately
 * quantized modules (codes [sum N_i, K/2], scales [sum N_i, K/16]); output column n of
 * segment i is scaled by that module's own global scale w_globals[i]:
 *   Y[:, off_i : off_i + N_i] = A . W_i^T,  off_i = N_0 + ... + N_{i-1}.
 * One launch; one shared activation quantization.  This is the repair of the global-scale
 * mismatch: a kernel that applied one scale to every segment would mis-scale segment i by
 * w_globals[0] / w_globals[i].
 *   1 <= num_segments <= NVFP4_MAX_SEGMENTS; seg_n (host) widths, each > 0.
 *   w_globals     device [num_segments].
 *   Other arguments as in nvfp4_gemm, with N = sum of seg_n.
 */
int nvfp4_gemm_fused_segments(int64_t M, int64_t K,
                              const uint8_t* a_codes, const uint8_t* a_scales,
                              const float* a_global, int a_global_per_row,
                              int num_segments, const int64_t* seg_n,
                              const uint8_t* w_codes, const uint8_t* w_scales,
                              const float* w_globals,
                              void* y, int y_dtype, int64_t ldy,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The (fused-module) GEMM with its output quantized to NVFP4 for the next linear layer, in
 * the same launch: Y is never written in bf16 or fp32.  Every linear layer takes 4-bit
 * activations ("Why Gated DeltaNet Survives 4-Bit Quantization", "The deep dive"), so a layer
 * whose output feeds another linear layer can hand it over already quantized.  For every output element the fp32
 * value y = (acc * a_global[m or 0]) * w_globals[seg(n)] is the one nvfp4_gemm_fused_segments
 * would store as fp32 for the same shape; each 16-column block of an output row is then
 * encoded exactly as nvfp4_quantize in NVFP4_SCALE_GIVEN mode encodes it under
 * y_global[0] (block max -> E4M3 scale -> E2M1 round-to-nearest-even).  The output global
 * scale is given (a calibrated, static scale): a dynamic per-tensor scale would need the
 * whole output before the first block could be encoded.  Format and encoding as for
 * nvfp4_quantize (sources in the file header).
 *   N = sum of seg_n, a multiple of 16; K a multiple of 128 below 2^24, and for M > 16 a
 *   multiple of 256 (other shapes: NVFP4_ERR_UNSUPPORTED).
 *   y_global      device [1], in: finite and > 0.
 *   y_codes       out [M, N/2], 16-byte aligned; y_scales out [M, N/16], 16-byte aligned.
 *   Other arguments as in nvfp4_gemm_fused_segments (one segment: a plain GEMM).
 */
int nvfp4_gemm_nvfp4_out(int64_t M, int64_t K,
                         const uint8_t* a_codes, const uint8_t* a_scales,
                         const float* a_global, int a_global_per_row,
                         int num_segments, const int64_t* seg_n,
                         const uint8_t* w_codes, const uint8_t* w_scales,
                         const float* w_globals,
                         const float* y_global, uint8_t* y_codes, uint8_t* y_scales,
                         void* stream);

/*
 * The fused Gated DeltaNet (GDN) input projection with its gate epilogue, in one launch.  The
 * GDN block has two gate projections, one setting how strongly the recurrent state is written
 * and one how much of it decays per step; the write strength goes through a sigmoid and the
 * decay is parameterized in log space through softplus and exponential ("Why Gated DeltaNet
 * Survives 4-Bit Quantization" (kipquest), "The deep dive", incl. its scope paragraph;
 * "Quantizing All Layers Reveals Recurrent Memory Is Robust" (freegardner), "The Gates That
 * Were Supposed to Break").  The pages print no formula; this is the standard GDN gate
 * parameterization that matches their description.
 * The last two segments are the gate projections, of equal width H (one column per value
 * head): the write-strength projection b, then the decay projection a.  Y is written exactly
 * as nvfp4_gemm_fused_segments writes it (all N columns, gate pre-activations included); in
 * addition, from each gate column's fp32 value y (before any rounding to y_dtype), for row m
 * and head j:
 *   beta[m, j] = 1 / (1 + exp(-y_b[m, j]))                           (write strength)
 *   g[m, j]    = -exp(a_log[j]) * softplus(y_a[m, j] + dt_bias[j])   (log decay; decay = e^g)
 * with softplus(z) = ln(1 + e^z), evaluated in fp32 without overflow.
 *   2 <= num_segments <= NVFP4_MAX_SEGMENTS, seg_n[num_segments-2] == seg_n[num_segments-1] = H.
 *   a_log, dt_bias  device [H] fp32, 4-byte aligned (per-head parameters).
 *   g, beta         device out [M, H] fp32, row-major, contiguous, 4-byte aligned.
 *   Other arguments as in nvfp4_gemm_fused_segments.
 */
int nvfp4_gemm_fused_gdn_gates(int64_t M, int64_t K,
                               const uint8_t* a_codes, const uint8_t* a_scales,
                               const float* a_global, int a_global_per_row,
                               int num_segments, const int64_t* seg_n,
                               const uint8_t* w_codes, const uint8_t* w_scales,
                               const float* w_globals,
                               void* y, int y_dtype, int64_t ldy,
                               const float* a_log, const float* dt_bias, float* g, float* beta,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace the GEMM entry points need for this shape: 0 for every shape at
 * present (decode reduces K inside the workgroup); kept so the ABI need not change. */
size_t nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * Lossy re-encoding of an NVFP4 tensor to MXFP4, the block-scaled 4-bit format that gfx950's
 * scaled FP4 matrix instructions take: E2M1 codes with one E8M0 scale (a power of two,
 * 2^(byte - 127)) per 32 consecutive elements of a row (OCP Microscaling (MX) specification
 * v1.0).  Each 32-element block (two NVFP4 blocks) is re-encoded from its exact NVFP4 values
 * v = E2M1 * E4M3 (the NVFP4 element format: "NVFP4 W4A4 Quantization Compresses 27B Hybrid
 * Models", "Challenging the Recurrence Fragility Assumption"), leaving the tensor's global
 * scale aside (it stays the multiplier of the MXFP4 tensor, unchanged):
 *   e = floor(log2(max |v|)) - 2 (the MX specification's shared exponent for E2M1),
 *   mx_scales byte = e + 127,  magnitude = E2M1_RNE_SAT(|v| / 2^e),  sign bit kept;
 *   a block of zeros gets byte 0 and magnitude 0.
 * Lossy by design: the E4M3 mantissa of each block scale is dropped and both 16-element halves
 * share one power-of-two scale.
 *   cols > 0 and a multiple of 32; rows >= 0 (0 is a no-op).
 *   codes     [rows, cols/2] NVFP4 codes, 16-byte aligned;  scales [rows, cols/16] E4M3, 2-byte aligned.
 *   mx_codes  out [rows, cols/2], 16-byte aligned (may be codes itself: in place);
 *   mx_scales out [rows, cols/32] E8M0 bytes.
 */
int nvfp4_to_mxfp4(int64_t rows, int64_t cols, const uint8_t* codes, const uint8_t* scales,
                   uint8_t* mx_codes, uint8_t* mx_scales, void* stream);

/*
 * The (fused-module) GEMM on MXFP4 operands with the scaled FP4 MFMA (fp32 accumulation):
 *   Y[m, n] = (sum_k E2M1(a_mk) 2^(sa_m,k/32 - 127) E2M1(w_nk) 2^(sw_n,k/32 - 127))
 *             * a_global[m or 0] * w_globals[seg(n)],
 * stored as fp32 or bf16 (round to nearest even).  Operands as nvfp4_to_mxfp4 writes them;
 * the global scales are the NVFP4 tensors' own.  With the operands re-encoded from NVFP4 this
 * is a lossy variant of nvfp4_gemm_fused_segments.
 *   K a multiple of 256 below 2^24 (other K: NVFP4_ERR_UNSUPPORTED); any M >= 0 (M <= 16 runs
 *   a decode kernel that streams W).  a_scales [M, K/32], w_scales [N, K/32], 16-byte aligned.
 *   Other arguments as in nvfp4_gemm_fused_segments (one segment: a plain GEMM).
 */
int nvfp4_mxfp4_gemm(int64_t M, int64_t K,
                     const uint8_t* a_codes, const uint8_t* a_scales,
                     const float* a_global, int a_global_per_row,
                     int num_segments, const int64_t* seg_n,
                     const uint8_t* w_codes, const uint8_t* w_scales,
                     const float* w_globals,
                     void* y, int y_dtype, int64_t ldy, void* stream);

/*
 * Interleave the gate and up projections of a gated (SwiGLU) MLP into the weight layout
 * nvfp4_gemm_swiglu takes: rows 32p .. 32p+15 of w are gate rows 16p .. 16p+15 and rows
 * 32p+16 .. 32p+31 the up rows 16p .. 16p+15 (codes and scale bytes alike), so that each
 * 32-row group holds both projections of 16 hidden units.  A one-time weight preparation (a
 * pure row permutation, stream-ordered device-to-device copies); the two projections keep
 * their own global scales, passed to nvfp4_gemm_swiglu as {gate, up}.
 *   F > 0 and a multiple of 16 (hidden width); K > 0 and a multiple of 16.
 *   gate_codes, up_codes    [F, K/2];  gate_scales, up_scales [F, K/16]   (device, contiguous).
 *   w_codes  out [2F, K/2];  w_scales out [2F, K/16]  (device, contiguous; must not overlap
 *   the inputs).
 */
int nvfp4_interleave_gate_up(int64_t F, int64_t K,
                             const uint8_t* gate_codes, const uint8_t* gate_scales,
                             const uint8_t* up_codes, const uint8_t* up_scales,
                             uint8_t* w_codes, uint8_t* w_scales, void* stream);

/*
 * The gated MLP input projection in one launch: the fused gate+up GEMM of the quantized
 * feed-forward block (paper abstract: NVFP4 W4A4 on all linear layers; "Why Gated DeltaNet
 * Survives 4-Bit Quantization", "The deep dive") with its SwiGLU activation and, optionally,
 * the NVFP4 encoding of the result for the down projection.  The pages do not name the MLP's
 * activation; this is the gated SiLU (SwiGLU) block of the Qwen family:
 *   y_gate[m, j], y_up[m, j] = the fp32 GEMM outputs (acc * a_global[m or 0]) * w_globals[0
 *   or 1] of hidden unit j, as nvfp4_gemm_fused_segments computes them for the segments
 *   [gate, up];
 *   h[m, j] = silu(y_gate) * y_up,  silu(y) = y * sigmoid(y) = y / (1 + e^-y)  (fp32).
 * h is stored as fp32 or bf16 (round to nearest even) when h is given, and as NVFP4 when
 * h_codes is given: each 16-element block of a row encoded exactly as nvfp4_quantize in
 * NVFP4_SCALE_GIVEN mode encodes it under h_global[0] (a calibrated, static scale).  At least
 * one of the two outputs is required.
 *   F > 0, a multiple of 16 (hidden width); K a multiple of 128 below 2^24, and for M > 16 a
 *   multiple of 256 (other shapes: NVFP4_ERR_UNSUPPORTED); M * F < 2^31.
 *   w_codes [2F, K/2], w_scales [2F, K/16]: the interleaved layout of nvfp4_interleave_gate_up.
 *   w_globals device [2] = {gate, up}.
 *   h       out [M, F] of h_dtype, row pitch ldh >= F elements, or NULL.
 *   h_global device [1], finite and > 0; h_codes out [M, F/2], h_scales out [M, F/16], both
 *   16-byte aligned; all three NULL when no NVFP4 output is wanted.
 *   Other arguments as in nvfp4_gemm.
 */
int nvfp4_gemm_swiglu(int64_t M, int64_t F, int64_t K,
                      const uint8_t* a_codes, const uint8_t* a_scales,
                      const float* a_global, int a_global_per_row,
                      const uint8_t* w_codes, const uint8_t* w_scales, const float* w_globals,
                      void* h, int h_dtype, int64_t ldh,
                      const float* h_global, uint8_t* h_codes, uint8_t* h_scales, void* stream);

/*
 * FP8 key-value cache codec with a calibrated per-tensor scale (the pages' second serving
 * finding: calibrated FP8 KV-cache scales are performance-free -- paper abstract;
 * "Quantizing All Layers Reveals Recurrent Memory Is Robust", "The Calibrated Cache That
 * Ships for Free"; "NVFP4 W4A4 Quantization Compresses 27B Hybrid Models", "Efficiency Gains
 * and Serving Optimization").  FP8 is the OCP E4M3FN byte of the file header; the tensor is
 * treated as n contiguous elements (e.g. a K or V cache flattened).
 *   quantize:   q[i] = sign | E4M3_RNE_SAT(fl32(|x[i]| / scale[0])) (round to nearest even,
 *               saturating at 448; +-inf -> +-448; NaN -> 0x7F).
 *   dequantize: y[i] = fl32(E4M3(q[i]) * scale[0]) as y_dtype (bf16: round to nearest even);
 *               0x7F / 0xFF -> NaN.
 *   x             [n] of x_dtype, 16-byte aligned.   q   [n] bytes, 8-byte aligned.
 *   y             [n] of y_dtype, 16-byte aligned.   scale device [1], finite and > 0.
 *   n >= 0        n == 0 is a no-op.
 */
int nvfp4_fp8_kv_quantize(const void* x, int x_dtype, int64_t n, const float* scale, uint8_t* q,
                          void* stream);
int nvfp4_fp8_kv_dequantize(const uint8_t* q, int64_t n, const float* scale, void* y, int y_dtype,
                            void* stream);

/* Static description of a status code. */
const char* nvfp4_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
