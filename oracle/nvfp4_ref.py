"""CPU oracle for NVFP4 W4A4: quantize, dequantize, block-scaled GEMM, fused segments.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
(``nvfp4_w4a4_block_amd``) never imports it, shares no code, tables or constants with it,
and must fail loudly rather than fall back to it.

It is written for being checked by eye, not for speed: plain numpy steps in the order the
format defines them, float32 where the format's arithmetic is binary32, float64 for the
GEMM.

Sources (the pages this follows):
  * "NVFP4 W4A4 Quantization Compresses 27B Hybrid Models" (thevalue.engineering), section
    "Challenging the Recurrence Fragility Assumption": NVFP4 = E2M1 4-bit element values
    with one E4M3 scale per 16-element block.
  * "Why Gated DeltaNet Survives 4-Bit Quantization" (kipquest paper page), "The deep dive":
    four-bit storage with one shared scale per sixteen-element block; W4A4 (weights and
    activations both four-bit) on every linear layer; block scaling confines an outlier to
    its own block of sixteen.
  * The paper abstract (Lattice and kipquest pages): modules that were calibrated one by one
    but run together as a single fused GEMM lose accuracy when the kernel applies one global
    scale to all of them, and the authors repair that.  A per-module global scale is
    therefore part of the format; each fused segment keeps its own.

Readings where the pages are silent (each is listed with its justification in the design
notes of this repository):
  R1 E2M1 magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code = sign<<3 | magnitude index.
  R2 E4M3 is the OCP E4M3FN byte (bias 7, no infinities, 0x7F/0xFF NaN, max 448).
  R3 Global scale s_g = fl32(amax / 2688), 2688 = 6 * 448 (largest E2M1 times largest E4M3),
     applied as a multiplier on dequantization.  Modes: one per tensor, one per row, or
     given by the caller.
  R4 Block scale byte s_j = E4M3_RNE_SAT(fl32(a_j / fl32(6 * s_g))), a_j = block max |x|.
  R5 Element: d_j = fl32(E4M3(s_j) * s_g); magnitude = E2M1_RNE_SAT(fl32(|x| / d_j)), or 0
     when d_j == 0; the sign bit is copied from x (so -0 and small negatives give code 8).
  R6 Ties go to the even code/byte (round to nearest even) in both E2M1 and E4M3; anything
     above the largest value saturates to it (6 for E2M1, 448 for E4M3).
  R7 Packing: two codes per byte, even column in the low nibble; scales one byte per block,
     row-major; both GEMM operands K-major (Y = A . W^T).
  R8 Dequantized value = E2M1(code) * E4M3(s_j) * s_g (exact in float64).
  R9 A tensor (per-tensor mode) or row (per-row mode) holding a NaN or an infinity has a
     non-finite global scale; its codes and scales are unspecified and not compared.

FP8 KV-cache codec (the pages' second serving finding: calibrated FP8 key-value cache scales
are performance-free -- paper abstract; "Quantizing All Layers Reveals Recurrent Memory Is
Robust" (freegardner), "The Calibrated Cache That Ships for Free"; "NVFP4 W4A4 Quantization
Compresses 27B Hybrid Models", "Efficiency Gains and Serving Optimization"):
  R10 FP8 is the OCP E4M3FN byte of R2; one calibrated scale s per tensor (K and V each),
      given by the caller.
  R11 Quantize: byte = sign | E4M3_RNE_SAT(fl32(|x| / s)) (the binary32 quotient, then R6);
      +-inf saturates to +-448, NaN gives 0x7F (the sign of a NaN quotient is not portable).
  R12 Dequantize: fl32(E4M3(byte) * s) (one binary32 rounding), NaN for 0x7F/0xFF.

Gated DeltaNet gate epilogue (the two gate projections of a GDN block, one controlling how
much of the recurrent state decays per step and one how strongly it is written; their
parameterization squashes GEMM error -- paper abstract, finding (ii); "Why Gated DeltaNet
Survives 4-Bit Quantization" (kipquest), "The deep dive"; "Quantizing All Layers Reveals
Recurrent Memory Is Robust" (freegardner), "The Gates That Were Supposed to Break": the
gates use softplus, exponential and sigmoid; the deep dive's scope paragraph: the decay is
parameterized in log space through softplus and exponential):
  R13 The fused GDN input projection ends with two segments of equal width H (one column
      per value head): the write-strength projection b, then the decay projection a.  Per
      head h: write strength beta = sigmoid(y_b) = 1 / (1 + e^-y_b); log-space decay
      g = -exp(A_log[h]) * softplus(y_a + dt_bias[h]), softplus(z) = ln(1 + e^z); decay
      factor alpha = e^g in (0, 1].  A_log and dt_bias are per-head float32 parameters.
      (The pages name the functions but print no formula; this is the standard Gated
      DeltaNet / Mamba-2 gate parameterization that matches their description.)
  R14 The gates take the GEMM's float32 output value y (global scales applied, R8 and the
      fused-segment repair) before any output rounding; g and beta are float32.

Lossy NVFP4 -> MXFP4 re-encoding (the pages' format is NVFP4 only -- "NVFP4 W4A4
Quantization Compresses 27B Hybrid Models", "Challenging the Recurrence Fragility
Assumption"; MXFP4 is the OCP Microscaling (MX) v1.0 format that gfx950's scaled FP4 matrix
instructions take; its definition here follows that published specification):
  R15 MXFP4: E2M1 codes (R1, packed as R7) with one E8M0 scale byte per 32 consecutive
      elements of a row (value 2^(byte - 127); 0xFF is NaN and never produced); the NVFP4
      tensor's float32 global scale is carried over unchanged and stays a multiplier.
  R16 A 32-element block (two NVFP4 blocks) is re-encoded from its exact NVFP4 values
      v = E2M1 * E4M3 (global scale left out): shared exponent e = floor(log2(max|v|)) - 2
      (2 = exponent of E2M1's largest power of two), scale 2^e, element magnitude
      E2M1_RNE_SAT(|v| / 2^e) (R6: ties to even, saturating at 6), the sign bit copied from
      the NVFP4 code.  A block of zeros gets scale byte 0 and magnitude 0.
  R17 The MXFP4 GEMM is the same contraction as R8's with the MXFP4 values
      E2M1 * 2^(byte - 127) * s_g.

Gated MLP input projection (the quantized feed-forward linears of the 27B hybrid model: paper
abstract, "all 496 linear layers"; "Why Gated DeltaNet Survives 4-Bit Quantization"
(kipquest), "The deep dive": W4A4 on every linear, feed-forward layers included).  The pages
do not name the MLP's activation:
  R18 The MLP is gated with SiLU (SwiGLU, the Qwen family's feed-forward block): the gate and
      up projections are two segments of one fused module, each with its own global scale,
      and the hidden activation is h = silu(y_gate) * y_up, silu(y) = y * sigmoid(y), taken
      from the GEMM's float32 outputs (global scales applied) before any output rounding.
      When h feeds the next linear (the down projection) it is encoded as NVFP4 under a
      given global scale, each 16-element block exactly as ``quantize`` in GIVEN mode.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32
F64 = np.float64

BLOCK = 16                         # elements per E4M3 block scale (R7, deep dive)
E2M1_MAX = 6.0                     # largest E2M1 magnitude (R1)
E4M3_MAX = 448.0                   # largest finite E4M3FN value (R2)
GLOBAL_DIVISOR = F32(E2M1_MAX * E4M3_MAX)   # 2688 (R3)

PER_TENSOR = "per_tensor"
PER_ROW = "per_row"
GIVEN = "given"

# R1: the eight E2M1 magnitudes, indexed by the 3-bit magnitude field.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=F64)

_CHUNK = 1 << 22


# ------------------------------------------------------------------------------ E2M1

def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit code (float64): sign bit 3, magnitude index bits 0..2 (R1)."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_rne_sat(v) -> np.ndarray:
    """Magnitude index (0..7) of the E2M1 value nearest to v >= 0; ties to the even index,
    values above 6 saturate to 6 (R6).  v is float32 (or anything exactly float64)."""
    v = np.asarray(v, dtype=F64)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    for s in range(0, flat.size, _CHUNK):
        c = flat[s:s + _CHUNK]
        dist = np.abs(c[:, None] - E2M1_MAGNITUDES[None, :])   # exact for float32 inputs
        best = dist.min(axis=1, keepdims=True)
        at_min = dist == best
        first = np.argmax(at_min, axis=1)                      # lowest nearest index
        nxt = np.minimum(first + 1, 7)
        tie = at_min[np.arange(c.size), nxt] & (nxt != first)
        # A tie is between two neighbouring indices; keep the even one.
        idx = np.where(tie & (first % 2 == 1), nxt, first)
        idx = np.where(c >= E2M1_MAX, 7, idx)                  # includes +inf
        out[s:s + c.size] = idx
    return out.reshape(v.shape)


# ------------------------------------------------------------------------------ E4M3

def e4m3_decode(b) -> np.ndarray:
    """Value of each E4M3FN byte (float64): sign bit 7, exponent bits 3..6 (bias 7),
    mantissa bits 0..2; exponent 0 is subnormal (m * 2^-9); 0x7F and 0xFF are NaN (R2)."""
    b = np.asarray(b).astype(np.int64)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(F64)))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return np.where((b & 0x80) != 0, -mag, mag)


# Non-negative finite E4M3 values; position in this table equals the byte (0x00..0x7E),
# and the table is increasing.
E4M3_TABLE = e4m3_decode(np.arange(0x7F))


def e4m3_rne_sat(t) -> np.ndarray:
    """Byte of the E4M3 value nearest to t >= 0; ties to the even byte (even mantissa);
    t above 448 (including +inf) saturates to 448 = 0x7E (R4, R6)."""
    t = np.asarray(t, dtype=F64)
    flat = t.reshape(-1)
    i = np.searchsorted(E4M3_TABLE, flat, side="right") - 1     # largest value <= t
    i = np.clip(i, 0, 0x7E)
    j = np.minimum(i + 1, 0x7E)
    lo = E4M3_TABLE[i]
    hi = E4M3_TABLE[j]
    d_lo = flat - lo        # exact: lo <= t and t, lo are within a factor of two or lo = 0
    d_hi = hi - flat
    up = (j != i) & ((d_hi < d_lo) | ((d_hi == d_lo) & (j % 2 == 0)))
    out = np.where(up, j, i)
    out = np.where(flat >= E4M3_MAX, 0x7E, out)
    return out.reshape(t.shape).astype(np.uint8)


# ------------------------------------------------------------------------------ tensors

@dataclass
class NVFP4:
    """An NVFP4 tensor: codes [R, C/2] (two per byte, even column low), E4M3 block scales
    [R, C/16], float32 global scale of shape (1,) or (R,), logical shape (R, C)."""
    codes: np.ndarray
    scales: np.ndarray
    global_scale: np.ndarray
    rows: int
    cols: int
    nonfinite: bool = False

    def global_per_row(self) -> np.ndarray:
        g = np.asarray(self.global_scale, dtype=F32).reshape(-1)
        return np.broadcast_to(g if g.size == self.rows else g[:1], (self.rows,))


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[R, C/2] bytes -> [R, C] 4-bit codes (R7: even column from the low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def pack_codes(code: np.ndarray) -> np.ndarray:
    """[R, C] 4-bit codes -> [R, C/2] bytes (R7)."""
    code = np.asarray(code, dtype=np.uint8)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)


def global_scale(x: np.ndarray, mode: str, given: float | None = None) -> np.ndarray:
    """R3: s_g = fl32(amax / 2688) over the tensor or each row, or the caller's value."""
    ax = np.abs(np.asarray(x, dtype=F32))
    if mode == PER_TENSOR:
        amax = ax.max() if ax.size else F32(0)
        return (np.asarray([amax], dtype=F32) / GLOBAL_DIVISOR).astype(F32)
    if mode == PER_ROW:
        amax = ax.max(axis=1) if ax.shape[1] else np.zeros(ax.shape[0], F32)
        return (amax.astype(F32) / GLOBAL_DIVISOR).astype(F32)
    if mode == GIVEN:
        return np.asarray([given], dtype=F32)
    raise ValueError(f"unknown mode {mode!r}")


def quantize(x, mode: str = PER_TENSOR, given: float | None = None) -> NVFP4:
    """Quantize X[R, C] (float32 values; bf16 inputs widened exactly) to NVFP4.

    Steps R3-R7 in order; all element arithmetic is binary32 with round-to-nearest-even.
    """
    x = np.ascontiguousarray(x, dtype=F32)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    R, C = x.shape
    if C % BLOCK:
        raise ValueError("cols must be a multiple of 16")
    nonfinite = not bool(np.isfinite(x).all())
    sg = global_scale(x, mode, given)                                   # (1,) or (R,)
    sg_row = np.broadcast_to(sg if sg.size == R else sg[:1], (R,)).astype(F32)[:, None]

    ax = np.abs(x).reshape(R, C // BLOCK, BLOCK)
    a = ax.max(axis=2) if C else np.zeros((R, 0), F32)                  # block max |x|
    with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
        den = (F32(E2M1_MAX) * sg_row).astype(F32)                      # fl32(6 * s_g)
        t = (a / den).astype(F32)                                       # fl32(a_j / den)
        s = e4m3_rne_sat(np.where(np.isnan(t), 0.0, t))
        s = np.where(sg_row == 0, 0, s).astype(np.uint8)                # zero tensor/row
        d = (e4m3_decode(s).astype(F32) * sg_row).astype(F32)           # fl32(E4M3(s) * s_g)
        q = (ax / d[:, :, None]).astype(F32)                            # fl32(|x| / d_j)
    mag = e2m1_rne_sat(np.where(np.isnan(q), 0.0, q))
    mag = np.where(d[:, :, None] == 0, 0, mag).reshape(R, C)
    sign = np.signbit(x).astype(np.int64)
    code = ((sign << 3) | mag).astype(np.uint8)
    return NVFP4(pack_codes(code), s, sg.astype(F32), R, C, nonfinite)


def dequantize(t: NVFP4, rows=None) -> np.ndarray:
    """R8: float64 values E2M1(code) * E4M3(scale) * s_g (exact), optionally for a subset
    of rows."""
    codes, scales, g = t.codes, t.scales, t.global_per_row()
    if rows is not None:
        rows = np.asarray(rows)
        codes, scales, g = codes[rows], scales[rows], g[rows]
    v = e2m1_decode(unpack_codes(codes))
    s = np.repeat(e4m3_decode(scales), BLOCK, axis=1)
    return v * s * g.astype(F64)[:, None]


def dequantize_f32(t: NVFP4) -> np.ndarray:
    """Binary32 dequantization fl32(E2M1 * fl32(E4M3 * s_g)), used to re-quantize."""
    v = e2m1_decode(unpack_codes(t.codes)).astype(F32)
    g = t.global_per_row().astype(F32)[:, None]
    d = (e4m3_decode(t.scales).astype(F32) * g).astype(F32)
    return (v * np.repeat(d, BLOCK, axis=1)).astype(F32)


# ------------------------------------------------------------------------------ GEMM

def gemm(a: NVFP4, w: NVFP4, a_rows=None):
    """Y[m, n] = sum_k A^[m, k] * W^[n, k] in float64 (Y = A^ . W^T), and the tolerance scale
    T[m, n] = sum_k |A^[m, k] * W^[n, k]|.  A^ and W^ are the exact dequantized operands
    (global scales included).  ``a_rows`` restricts to a subset of output rows."""
    if a.cols != w.cols:
        raise ValueError("K mismatch")
    A = dequantize(a, a_rows)
    W = dequantize(w)
    return A @ W.T, np.abs(A) @ np.abs(W).T


def fused_segments(a: NVFP4, segments: list[NVFP4], a_rows=None):
    """The repaired fused GEMM: output columns of segment i are A^ . W_i^T with W_i
    dequantized under its own global scale; segments are concatenated along N."""
    ys, ts = zip(*(gemm(a, w, a_rows) for w in segments))
    return np.concatenate(ys, axis=1), np.concatenate(ts, axis=1)


def fused_shared_scale(a: NVFP4, segments: list[NVFP4], shared: float, a_rows=None):
    """The global-scale mismatch (negative control): the fused launch dequantizes every
    segment's codes and block scales with one shared global scale instead of its own."""
    relabeled = [NVFP4(w.codes, w.scales, np.asarray([shared], F32), w.rows, w.cols)
                 for w in segments]
    return fused_segments(a, relabeled, a_rows)


def nvfp4_bytes(rows: int, cols: int, global_scales: int = 1) -> int:
    """Storage of one NVFP4 tensor: 4-bit codes + one byte per 16 elements + fp32 scales."""
    return rows * cols // 2 + rows * cols // BLOCK + 4 * global_scales


# ------------------------------------------------------------------------------ FP8 KV cache

def fp8_kv_quantize(x, scale: float) -> np.ndarray:
    """FP8 (E4M3FN) bytes of x under the calibrated per-tensor scale s (R10, R11): the
    binary32 quotient x / s, rounded to the nearest E4M3 value (ties to even), saturating at
    448; the sign bit is copied (so -0 gives 0x80); NaN gives 0x7F."""
    x32 = np.asarray(x, dtype=F32)
    t = (x32 / F32(scale)).astype(F32)                      # IEEE binary32 division
    sign = np.where(np.signbit(t), 0x80, 0).astype(np.uint8)
    a = np.abs(t).astype(F64)
    nan = np.isnan(a)
    mag = e4m3_rne_sat(np.where(nan, 0.0, a))
    return np.where(nan, 0x7F, mag | sign).astype(np.uint8)


def fp8_kv_dequantize(q, scale: float) -> np.ndarray:
    """fl32(E4M3(byte) * s) (R12): the product of two binary32 numbers is exact in float64,
    so one rounding to float32 gives the binary32 product."""
    v = e4m3_decode(np.asarray(q, dtype=np.uint8))
    return (v * F64(F32(scale))).astype(F32)


# ------------------------------------------------------------------------------ GDN gates

def sigmoid(y) -> np.ndarray:
    """1 / (1 + e^-y) in float64 (R13), in the form that never overflows: e^-|y| is at most
    1, and for y < 0 the value is e^y / (1 + e^y)."""
    y = np.asarray(y, dtype=F64)
    e = np.exp(-np.abs(y))
    return np.where(y >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(z) -> np.ndarray:
    """ln(1 + e^z) in float64 (R13), as max(z, 0) + ln(1 + e^-|z|), which is the same
    number without overflow for large z or loss of e^z for very negative z."""
    z = np.asarray(z, dtype=F64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def gdn_gates(y_b, y_a, a_log, dt_bias):
    """R13: (g, beta) for pre-activations y_b, y_a of shape [M, H] and per-head A_log,
    dt_bias of shape [H]: beta = sigmoid(y_b), g = -exp(A_log) * softplus(y_a + dt_bias).
    Float64 throughout; the parameters are float32 values widened exactly."""
    a_log = np.asarray(a_log, dtype=F32).astype(F64)
    dt = np.asarray(dt_bias, dtype=F32).astype(F64)
    beta = sigmoid(y_b)
    g = -np.exp(a_log)[None, :] * softplus(np.asarray(y_a, dtype=F64) + dt[None, :])
    return g, beta


def fused_gdn_gates(a: NVFP4, segments: list[NVFP4], a_log, dt_bias, a_rows=None):
    """The fused GDN input projection with its gate epilogue (R13, R14): Y and T over all
    segments exactly as ``fused_segments``, and (g, beta) from the last two segments, which
    must have equal widths H (b, then a)."""
    if len(segments) < 2 or segments[-1].rows != segments[-2].rows:
        raise ValueError("the last two segments must be the two gate projections of equal width")
    Y, T = fused_segments(a, segments, a_rows)
    H = segments[-1].rows
    N = Y.shape[1]
    g, beta = gdn_gates(Y[:, N - 2 * H:N - H], Y[:, N - H:], a_log, dt_bias)
    return Y, T, g, beta


# ------------------------------------------------------------------------------ SwiGLU MLP input

def silu(y) -> np.ndarray:
    """y * sigmoid(y) in float64 (R18), with the overflow-free sigmoid above."""
    y = np.asarray(y, dtype=F64)
    return y * sigmoid(y)


def swiglu_mlp(a: NVFP4, gate: NVFP4, up: NVFP4, a_rows=None):
    """The gated MLP input projection (R18): Y_g = A^ . G^T and Y_u = A^ . U^T, each weight
    dequantized under its own global scale, and H = silu(Y_g) * Y_u, all float64.  Returns
    (H, Y_g, T_g, Y_u, T_u), the T being ``gemm``'s tolerance scales of the two products."""
    if gate.rows != up.rows:
        raise ValueError("the gate and up projections must have the same width")
    yg, tg = gemm(a, gate, a_rows)
    yu, tu = gemm(a, up, a_rows)
    return silu(yg) * yu, yg, tg, yu, tu


# ------------------------------------------------------------------------------ MXFP4 (lossy)

MX_BLOCK = 32                      # elements per E8M0 scale (R15)
E2M1_EMAX = 2                      # exponent of E2M1's largest power of two, 4 = 2^2 (R16)


@dataclass
class MXFP4:
    """An MXFP4 tensor: codes [R, C/2] (as NVFP4), E8M0 scale bytes [R, C/32], float32
    global scale of shape (1,) or (R,) carried over from the NVFP4 tensor."""
    codes: np.ndarray
    scales: np.ndarray
    global_scale: np.ndarray
    rows: int
    cols: int

    def global_per_row(self) -> np.ndarray:
        g = np.asarray(self.global_scale, dtype=F32).reshape(-1)
        return np.broadcast_to(g if g.size == self.rows else g[:1], (self.rows,))


def e8m0_decode(b) -> np.ndarray:
    """2^(byte - 127) as float64; 0xFF is NaN (R15)."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.exp2((b - 127).astype(F64)))


def mxfp4_from_nvfp4(t: NVFP4) -> MXFP4:
    """R16: re-encode each 32-element block of an NVFP4 tensor to MXFP4 (lossy)."""
    if t.cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    R, C = t.rows, t.cols
    code = unpack_codes(t.codes)
    v = e2m1_decode(code) * np.repeat(e4m3_decode(t.scales), BLOCK, axis=1)   # exact
    blocks = np.abs(v).reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = blocks.max(axis=2) if C else np.zeros((R, 0))
    # floor(log2(amax)) from the binary exponent: amax = m * 2^ex with 0.5 <= m < 1.
    _, ex = np.frexp(amax)
    shared = ex.astype(np.int64) - 1 - E2M1_EMAX
    zero = amax == 0
    shared = np.where(zero, -127, shared)
    q = blocks / np.exp2(shared.astype(F64))[:, :, None]                    # exact (power of 2)
    mag = e2m1_rne_sat(q).reshape(R, C)
    mag = np.where(np.repeat(zero, MX_BLOCK, axis=1), 0, mag)
    sign = (code >> 3) & 1
    out = ((sign << 3) | mag).astype(np.uint8)
    scales = (shared + 127).astype(np.uint8)
    return MXFP4(pack_codes(out), scales, np.asarray(t.global_scale, F32).copy(), R, C)


def mx_dequantize(t: MXFP4, rows=None) -> np.ndarray:
    """R17: float64 values E2M1(code) * 2^(byte - 127) * s_g (exact)."""
    codes, scales, g = t.codes, t.scales, t.global_per_row()
    if rows is not None:
        rows = np.asarray(rows)
        codes, scales, g = codes[rows], scales[rows], g[rows]
    v = e2m1_decode(unpack_codes(codes))
    s = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=1)
    return v * s * g.astype(F64)[:, None]


def mx_gemm(a: MXFP4, w: MXFP4, a_rows=None):
    """Y = A^ . W^T in float64 for MXFP4 operands, and T = |A^| . |W^|^T (R17)."""
    if a.cols != w.cols:
        raise ValueError("K mismatch")
    A = mx_dequantize(a, a_rows)
    W = mx_dequantize(w)
    return A @ W.T, np.abs(A) @ np.abs(W).T
