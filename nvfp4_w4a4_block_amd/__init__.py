"""Python binding of the MI355X NVFP4 W4A4 library (``libnvfp4.so``, C ABI in
``include/nvfp4.h``).

Argument marshalling only: every step of quantization and GEMM runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  If the library is not
built this module raises ImportError; there is no fallback implementation.

Entry points (same names as the C ABI):
  quantize(x, mode)                      -> NVFP4Tensor (codes, scales, global_scale)
  gemm(a, w, out_dtype)                  -> Y = A . W^T
  gemm_fused_segments(a, w, widths, w_globals, out_dtype)
                                         -> Y with one weight global scale per segment
  gemm_nvfp4_out(a, w_codes, w_scales, widths, w_globals, y_global)
                                         -> Y quantized to NVFP4 under a given global scale
  fp8_kv_quantize(x, scale) / fp8_kv_dequantize(q, scale, out_dtype)
                                         -> FP8 (E4M3) KV-cache codec, calibrated scale
  gemm_fused_gdn_gates(a, w_codes, w_scales, widths, w_globals, a_log, dt_bias, out_dtype)
                                         -> (Y, g, beta): fused GDN input projection whose
                                            last two segments leave as log decay and
                                            write strength
  to_mxfp4(a) / mxfp4_gemm(a_mx, w_codes, w_scales, widths, w_globals, out_dtype)
                                         -> lossy MXFP4 re-encoding and the GEMM on gfx950's
                                            scaled FP4 MFMA
  interleave_gate_up(gate, up)           -> (w_codes, w_scales): gate and up projections of a
                                            gated MLP in 16-row interleaved groups
  gemm_swiglu(a, w_codes, w_scales, w_globals, h_dtype, h_global)
                                         -> (h, h as NVFP4): the fused gate+up GEMM with its
                                            SwiGLU activation, h = silu(gate) * up
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Sequence

import torch

__all__ = [
    "NVFP4Tensor", "NVFP4Error", "quantize", "gemm", "gemm_fused_segments", "gemm_nvfp4_out", "gemm_fused_gdn_gates", "MXFP4Tensor", "to_mxfp4", "mxfp4_gemm",
    "fp8_kv_quantize", "fp8_kv_dequantize", "interleave_gate_up", "gemm_swiglu", "decode_linear",
    "library_path", "lib",
    "PER_TENSOR", "PER_ROW", "GIVEN", "MAX_SEGMENTS", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

PER_TENSOR, PER_ROW, GIVEN = 0, 1, 2
_MODES = {"per_tensor": PER_TENSOR, "per_row": PER_ROW, "given": GIVEN}
_F32, _BF16 = 0, 1
MAX_SEGMENTS = 64
EXPORTED_SYMBOLS = (
    "nvfp4_quantize", "nvfp4_quantize_workspace_size", "nvfp4_quantize_no_alloc", "nvfp4_gemm", "nvfp4_gemm_fused_segments",
    "nvfp4_gemm_nvfp4_out", "nvfp4_gemm_fused_gdn_gates", "nvfp4_to_mxfp4", "nvfp4_mxfp4_gemm",
    "nvfp4_gemm_workspace_size", "nvfp4_fp8_kv_quantize", "nvfp4_fp8_kv_dequantize",
    "nvfp4_interleave_gate_up", "nvfp4_gemm_swiglu", "nvfp4_decode_linear", "nvfp4_status_string",
    "nvfp4_version",
)


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python nvfp4_w4a4_block_amd/build.py`")
    L = ctypes.CDLL(_LIB_PATH)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.nvfp4_quantize.argtypes = [p, i32, i64, i64, i64, p, p, p, i32, p, sz, p]
    L.nvfp4_quantize.restype = i32
    L.nvfp4_quantize_no_alloc.argtypes = [p, i32, i64, i64, i64, p, p, p, i32, p]
    L.nvfp4_quantize_no_alloc.restype = i32
    L.nvfp4_quantize_workspace_size.argtypes = [i64, i64, i32]
    L.nvfp4_quantize_workspace_size.restype = sz
    L.nvfp4_gemm.argtypes = [i64, i64, i64, p, p, p, i32, p, p, p, p, i32, i64, p, sz, p]
    L.nvfp4_gemm.restype = i32
    L.nvfp4_decode_linear.argtypes = [i64, i64, p, i32, i32, p, p, p, p, p, p, p, i32, p]
    L.nvfp4_decode_linear.restype = i32
    L.nvfp4_gemm_fused_segments.argtypes = [i64, i64, p, p, p, i32, i32, p, p, p, p, p, i32, i64, p, sz, p]
    L.nvfp4_gemm_fused_segments.restype = i32
    L.nvfp4_gemm_nvfp4_out.argtypes = [i64, i64, p, p, p, i32, i32, p, p, p, p, p, p, p, p]
    L.nvfp4_gemm_nvfp4_out.restype = i32
    L.nvfp4_gemm_fused_gdn_gates.argtypes = [i64, i64, p, p, p, i32, i32, p, p, p, p, p, i32, i64, p, p, p, p,
                                             p, sz, p]
    L.nvfp4_gemm_fused_gdn_gates.restype = i32
    L.nvfp4_to_mxfp4.argtypes = [i64, i64, p, p, p, p, p]
    L.nvfp4_to_mxfp4.restype = i32
    L.nvfp4_mxfp4_gemm.argtypes = [i64, i64, p, p, p, i32, i32, p, p, p, p, p, i32, i64, p]
    L.nvfp4_mxfp4_gemm.restype = i32
    L.nvfp4_fp8_kv_quantize.argtypes = [p, i32, i64, p, p, p]
    L.nvfp4_fp8_kv_quantize.restype = i32
    L.nvfp4_fp8_kv_dequantize.argtypes = [p, i64, p, p, i32, p]
    L.nvfp4_fp8_kv_dequantize.restype = i32
    L.nvfp4_interleave_gate_up.argtypes = [i64, i64, p, p, p, p, p, p, p]
    L.nvfp4_interleave_gate_up.restype = i32
    L.nvfp4_gemm_swiglu.argtypes = [i64, i64, i64, p, p, p, i32, p, p, p, p, i32, i64, p, p, p, p]
    L.nvfp4_gemm_swiglu.restype = i32
    L.nvfp4_gemm_workspace_size.argtypes = [i64, i64, i64]
    L.nvfp4_gemm_workspace_size.restype = sz
    L.nvfp4_status_string.argtypes = [i32]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_version.argtypes = []
    L.nvfp4_version.restype = i32
    return L


lib = _load()


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.nvfp4_status_string(status).decode()} (status {status})")


def _check(status: int, what: str) -> None:
    if status != 0:
        raise NVFP4Error(status, what)


@dataclass
class NVFP4Tensor:
    """codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], global_scale float32 [1] or
    [rows], all on one GPU."""
    codes: torch.Tensor
    scales: torch.Tensor
    global_scale: torch.Tensor

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1] * 2


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _require_bytes(t: torch.Tensor, shape: tuple, name: str, dev: torch.device) -> None:
    """A contiguous uint8 tensor of exactly ``shape`` on ``dev``: the library reads and writes
    codes and scale bytes at the pitch their width implies."""
    _require(isinstance(t, torch.Tensor) and t.device == dev, f"{name}: a tensor on {dev}")
    _require(t.dtype == torch.uint8 and t.is_contiguous(), f"{name}: contiguous uint8")
    _require(tuple(t.shape) == tuple(shape), f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _require_f32(t: torch.Tensor, numel: int | tuple, name: str, dev: torch.device) -> None:
    """A contiguous fp32 tensor on ``dev`` with ``numel`` elements (or one of several counts)."""
    counts = numel if isinstance(numel, tuple) else (numel,)
    _require(isinstance(t, torch.Tensor) and t.device == dev, f"{name}: a tensor on {dev}")
    _require(t.dtype == torch.float32 and t.is_contiguous(), f"{name}: contiguous float32")
    _require(t.numel() in counts, f"{name}: {t.numel()} elements, expected {' or '.join(map(str, counts))}")


def _require_operand(t, name: str, group: int = 16) -> None:
    """Codes [R, C/2] and scales [R, C/group] of one device, contiguous; the global scale is
    checked by the caller (its count depends on the role)."""
    _require(isinstance(t.codes, torch.Tensor) and t.codes.dim() == 2, f"{name}.codes: 2-D")
    dev = t.codes.device
    R, C = t.codes.shape[0], t.codes.shape[1] * 2
    _require_bytes(t.codes, (R, C // 2), f"{name}.codes", dev)
    _require_bytes(t.scales, (R, C // group), f"{name}.scales", dev)


def _on_gpu(dev: torch.device) -> None:
    """Checked last, after every shape and dtype check, so that those checks can be exercised
    on a machine without a GPU: every tensor of a call is on ``dev``, which must be a GPU."""
    _require(dev.type == "cuda", f"tensors must be on a GPU, not {dev}")


def _a_global_per_row(a) -> int:
    """1 when the activation carries one global scale per row, 0 for one per tensor; any
    other count is an error (a row slice of a per-row tensor must slice its scales too)."""
    M = a.rows
    _require_f32(a.global_scale, (1, M), "a.global_scale", a.codes.device)
    return int(a.global_scale.numel() == M and M != 1)


def quantize(x: torch.Tensor, mode: str = "per_tensor", global_scale: torch.Tensor | None = None,
             out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """Quantize a 2-D bf16/fp32 CUDA tensor (row stride may exceed its width) to NVFP4.

    mode: "per_tensor" | "per_row" | "given" (then ``global_scale`` is a float32 CUDA tensor
    of one element)."""
    _require(isinstance(x, torch.Tensor) and x.dim() == 2, "x must be a 2-D tensor")
    _require(x.dtype in (torch.bfloat16, torch.float32), "x must be bf16 or fp32")
    _require(x.stride(1) == 1 or x.shape[0] == 0, "x must be row-contiguous")   # (no rows: no data)
    _require(mode in _MODES, f"mode must be one of {sorted(_MODES)}")
    m = _MODES[mode]
    rows, cols = x.shape
    dev = x.device
    if out is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        if m == GIVEN:
            _require(global_scale is not None, "given mode needs global_scale")
            g = global_scale
        else:
            g = torch.empty((rows if m == PER_ROW else 1,), dtype=torch.float32, device=dev)
        out = NVFP4Tensor(codes, scales, g)
    elif m == GIVEN and global_scale is not None:
        out.global_scale = global_scale
    _require_bytes(out.codes, (rows, cols // 2), "out.codes", dev)
    _require_bytes(out.scales, (rows, cols // 16), "out.scales", dev)
    _require_f32(out.global_scale, rows if m == PER_ROW else 1, "global scale", dev)
    ws_bytes = lib.nvfp4_quantize_workspace_size(rows, cols, m)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev) if ws_bytes else None
    ldx = x.stride(0) if rows > 1 else max(x.stride(0), cols)
    _on_gpu(dev)
    st = lib.nvfp4_quantize(_ptr(x), _BF16 if x.dtype == torch.bfloat16 else _F32, rows, cols, ldx,
                            _ptr(out.codes), _ptr(out.scales), _ptr(out.global_scale), m,
                            _ptr(ws), ws_bytes, _stream(dev))
    _check(st, "nvfp4_quantize")
    return out


def _fused_weight_checks(a, w_codes: torch.Tensor, w_scales: torch.Tensor, seg_widths: Sequence[int],
                         w_globals: torch.Tensor, group: int = 16):
    """Shapes and devices of a (fused) weight: codes [N, K/2], scale bytes [N, K/group], one
    fp32 global scale per segment.  Returns (M, K, N, device)."""
    _require_operand(a, "a", group)
    M, K = a.rows, a.cols
    _require(len(seg_widths) >= 1 and all(int(v) > 0 for v in seg_widths), "segment widths must be positive")
    N = int(sum(int(v) for v in seg_widths))
    dev = a.codes.device
    _require_bytes(w_codes, (N, K // 2), "w_codes", dev)
    _require_bytes(w_scales, (N, K // group), "w_scales", dev)
    _require_f32(w_globals, len(seg_widths), "w_globals (one per segment)", dev)
    return M, K, N, dev


def _out_tensor(M: int, N: int, dtype: torch.dtype, dev, out: torch.Tensor | None) -> torch.Tensor:
    if out is None:
        return torch.empty((M, N), dtype=dtype, device=dev)
    _require(out.device == dev, f"out: a tensor on {dev}")
    _require(out.shape == (M, N) and out.dtype == dtype and out.stride(1) == 1, "bad out tensor")
    return out


def _y_dtype(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return _BF16
    _require(dtype == torch.float32, "out_dtype must be bfloat16 or float32")
    return _F32


def gemm(a: NVFP4Tensor, w: NVFP4Tensor, out_dtype: torch.dtype = torch.bfloat16,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] = A . W^T for NVFP4 A [M, K] and W [N, K]."""
    _require_operand(a, "a")
    _require_operand(w, "w")
    _require(a.cols == w.cols, "K mismatch")
    M, N, K = a.rows, w.rows, a.cols
    dev = a.codes.device
    _require(w.codes.device == dev, "a and w must be on one device")
    _require_f32(w.global_scale, 1, "w.global_scale (one per tensor)", dev)
    y = _out_tensor(M, N, out_dtype, dev, out)
    per_row = _a_global_per_row(a)
    ws_bytes = lib.nvfp4_gemm_workspace_size(M, N, K)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev) if ws_bytes else None
    _on_gpu(dev)
    st = lib.nvfp4_gemm(M, N, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.global_scale), per_row,
                        _ptr(w.codes), _ptr(w.scales), _ptr(w.global_scale), _ptr(y), _y_dtype(out_dtype),
                        y.stride(0) if M > 0 else N, _ptr(ws), ws_bytes, _stream(dev))
    _check(st, "nvfp4_gemm")
    return y


def decode_linear(x: torch.Tensor, w: NVFP4Tensor, mode: str = "per_tensor",
                  global_scale: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                  out: torch.Tensor | None = None, a_out: NVFP4Tensor | None = None):
    """Batch-1 decode of one linear layer: quantize the token x [1, K] (bf16 or fp32) and
    multiply with W [N, K] in one call.  Returns (y [1, N], the token as NVFP4); the same bits as
    ``quantize(x, mode, global_scale)`` followed by ``gemm``.  mode: "per_tensor" or "per_row"
    (the same scale for one row) or "given" (``global_scale``: one fp32 element)."""
    _require(isinstance(x, torch.Tensor) and x.dim() == 2 and x.shape[0] == 1, "x must be [1, K]")
    _require(x.dtype in (torch.bfloat16, torch.float32), "x must be bf16 or fp32")
    _require(x.is_contiguous(), "x must be contiguous")
    _require(mode in _MODES, f"mode must be one of {sorted(_MODES)}")
    _require_operand(w, "w")
    K, N, dev = x.shape[1], w.rows, x.device
    _require(w.cols == K, "K mismatch")
    _require(w.codes.device == dev, "x and w must be on one device")
    _require_f32(w.global_scale, 1, "w.global_scale (one per tensor)", dev)
    m = _MODES[mode]
    if a_out is None:
        if m == GIVEN:
            _require(global_scale is not None, "given mode needs global_scale")
            g = global_scale
        else:
            g = torch.empty((1,), dtype=torch.float32, device=dev)
        a_out = NVFP4Tensor(torch.empty((1, K // 2), dtype=torch.uint8, device=dev),
                            torch.empty((1, K // 16), dtype=torch.uint8, device=dev), g)
    elif m == GIVEN and global_scale is not None:
        a_out.global_scale = global_scale
    _require_bytes(a_out.codes, (1, K // 2), "a_out.codes", dev)
    _require_bytes(a_out.scales, (1, K // 16), "a_out.scales", dev)
    _require_f32(a_out.global_scale, 1, "a_out.global_scale", dev)
    y = _out_tensor(1, N, out_dtype, dev, out)
    _require(y.is_contiguous(), "out must be contiguous")
    _on_gpu(dev)
    st = lib.nvfp4_decode_linear(N, K, _ptr(x), _BF16 if x.dtype == torch.bfloat16 else _F32, m,
                                 _ptr(a_out.codes), _ptr(a_out.scales), _ptr(a_out.global_scale),
                                 _ptr(w.codes), _ptr(w.scales), _ptr(w.global_scale), _ptr(y),
                                 _y_dtype(out_dtype), _stream(dev))
    _check(st, "nvfp4_decode_linear")
    return y, a_out


def gemm_fused_segments(a: NVFP4Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
                        seg_widths: Sequence[int], w_globals: torch.Tensor,
                        out_dtype: torch.dtype = torch.bfloat16,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """Fused-module GEMM: W = concatenation (along N) of len(seg_widths) modules, each with its
    own global scale w_globals[i] (fp32 GPU tensor)."""
    M, K, N, dev = _fused_weight_checks(a, w_codes, w_scales, seg_widths, w_globals)
    y = _out_tensor(M, N, out_dtype, dev, out)
    per_row = _a_global_per_row(a)
    widths = (ctypes.c_int64 * len(seg_widths))(*[int(v) for v in seg_widths])
    ws_bytes = lib.nvfp4_gemm_workspace_size(M, N, K)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev) if ws_bytes else None
    _on_gpu(dev)
    st = lib.nvfp4_gemm_fused_segments(M, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.global_scale), per_row,
                                       len(seg_widths), ctypes.cast(widths, ctypes.c_void_p),
                                       _ptr(w_codes), _ptr(w_scales), _ptr(w_globals), _ptr(y),
                                       _y_dtype(out_dtype), y.stride(0) if M > 0 else N, _ptr(ws), ws_bytes,
                                       _stream(dev))
    _check(st, "nvfp4_gemm_fused_segments")
    return y


def gemm_nvfp4_out(a: NVFP4Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, seg_widths: Sequence[int],
                   w_globals: torch.Tensor, y_global: torch.Tensor,
                   out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """(Fused-module) GEMM whose output is quantized to NVFP4 in the same launch, under the
    given output global scale y_global (fp32 GPU tensor of one element).  With one segment
    it is a plain GEMM.  Returns NVFP4Tensor(codes [M, N/2], scales [M, N/16], y_global)."""
    M, K, N, dev = _fused_weight_checks(a, w_codes, w_scales, seg_widths, w_globals)
    _require_f32(y_global, 1, "y_global", dev)
    if out is None:
        out = NVFP4Tensor(torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
                          torch.empty((M, N // 16), dtype=torch.uint8, device=dev), y_global)
    _require_bytes(out.codes, (M, N // 2), "out.codes", dev)
    _require_bytes(out.scales, (M, N // 16), "out.scales", dev)
    per_row = _a_global_per_row(a)
    widths = (ctypes.c_int64 * len(seg_widths))(*[int(v) for v in seg_widths])
    _on_gpu(dev)
    st = lib.nvfp4_gemm_nvfp4_out(M, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.global_scale), per_row,
                                  len(seg_widths), ctypes.cast(widths, ctypes.c_void_p), _ptr(w_codes),
                                  _ptr(w_scales), _ptr(w_globals), _ptr(y_global), _ptr(out.codes),
                                  _ptr(out.scales), _stream(dev))
    _check(st, "nvfp4_gemm_nvfp4_out")
    return out


def gemm_fused_gdn_gates(a: NVFP4Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor,
                         seg_widths: Sequence[int], w_globals: torch.Tensor, a_log: torch.Tensor,
                         dt_bias: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                         out: torch.Tensor | None = None, g_out: torch.Tensor | None = None,
                         beta_out: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Fused GDN input projection with the gate epilogue in the same launch.  The last two
    segments (equal widths H) are the write-strength and decay projections; a_log and dt_bias
    are fp32 GPU tensors [H].  Returns (Y [M, N] as gemm_fused_segments writes it, g [M, H]
    fp32 log decay, beta [M, H] fp32 write strength)."""
    _require(len(seg_widths) >= 2 and seg_widths[-1] == seg_widths[-2], "the last two segments are the gates")
    M, K, N, dev = _fused_weight_checks(a, w_codes, w_scales, seg_widths, w_globals)
    H = int(seg_widths[-1])
    _require_f32(a_log, H, "a_log [H]", dev)
    _require_f32(dt_bias, H, "dt_bias [H]", dev)
    y = _out_tensor(M, N, out_dtype, dev, out)
    g = _out_tensor(M, H, torch.float32, dev, g_out)
    beta = _out_tensor(M, H, torch.float32, dev, beta_out)
    _require(g.is_contiguous() and beta.is_contiguous(), "g and beta must be contiguous")
    per_row = _a_global_per_row(a)
    widths = (ctypes.c_int64 * len(seg_widths))(*[int(v) for v in seg_widths])
    ws_bytes = lib.nvfp4_gemm_workspace_size(M, N, K)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev) if ws_bytes else None
    _on_gpu(dev)
    st = lib.nvfp4_gemm_fused_gdn_gates(M, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.global_scale), per_row,
                                        len(seg_widths), ctypes.cast(widths, ctypes.c_void_p), _ptr(w_codes),
                                        _ptr(w_scales), _ptr(w_globals), _ptr(y), _y_dtype(out_dtype),
                                        y.stride(0) if M > 0 else N, _ptr(a_log), _ptr(dt_bias), _ptr(g),
                                        _ptr(beta), _ptr(ws), ws_bytes, _stream(dev))
    _check(st, "nvfp4_gemm_fused_gdn_gates")
    return y, g, beta


@dataclass
class MXFP4Tensor:
    """codes uint8 [rows, cols/2] (E2M1, as NVFP4), scales uint8 [rows, cols/32] (E8M0),
    global_scale float32 [1] or [rows] (the NVFP4 tensor's), all on one GPU."""
    codes: torch.Tensor
    scales: torch.Tensor
    global_scale: torch.Tensor

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1] * 2


def to_mxfp4(t: NVFP4Tensor, out: MXFP4Tensor | None = None) -> MXFP4Tensor:
    """Lossy re-encoding of an NVFP4 tensor to MXFP4 (E8M0 scale per 32 elements); the global
    scale tensor is shared with the input."""
    _require_operand(t, "t")
    R, C = t.rows, t.cols
    _require(C % 32 == 0, "cols must be a multiple of 32")
    dev = t.codes.device
    if out is None:
        out = MXFP4Tensor(torch.empty((R, C // 2), dtype=torch.uint8, device=dev),
                          torch.empty((R, C // 32), dtype=torch.uint8, device=dev), t.global_scale)
    _require_bytes(out.codes, (R, C // 2), "out.codes", dev)
    _require_bytes(out.scales, (R, C // 32), "out.scales", dev)
    _on_gpu(dev)
    st = lib.nvfp4_to_mxfp4(R, C, _ptr(t.codes), _ptr(t.scales), _ptr(out.codes), _ptr(out.scales), _stream(dev))
    _check(st, "nvfp4_to_mxfp4")
    return out


def mxfp4_gemm(a: MXFP4Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, seg_widths: Sequence[int],
               w_globals: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """(Fused-module) GEMM on MXFP4 operands with the scaled FP4 MFMA: W = concatenation of the
    segments' MXFP4 codes [N, K/2] and E8M0 scales [N, K/32], one global scale per segment."""
    M, K, N, dev = _fused_weight_checks(a, w_codes, w_scales, seg_widths, w_globals, group=32)
    y = _out_tensor(M, N, out_dtype, dev, out)
    per_row = _a_global_per_row(a)
    widths = (ctypes.c_int64 * len(seg_widths))(*[int(v) for v in seg_widths])
    _on_gpu(dev)
    st = lib.nvfp4_mxfp4_gemm(M, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.global_scale), per_row, len(seg_widths),
                              ctypes.cast(widths, ctypes.c_void_p), _ptr(w_codes), _ptr(w_scales), _ptr(w_globals),
                              _ptr(y), _y_dtype(out_dtype), y.stride(0) if M > 0 else N, _stream(dev))
    _check(st, "nvfp4_mxfp4_gemm")
    return y


def interleave_gate_up(gate: NVFP4Tensor, up: NVFP4Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """The weight layout gemm_swiglu takes: rows 32p .. 32p+15 are gate rows 16p .. 16p+15,
    rows 32p+16 .. 32p+31 the up rows 16p .. 16p+15.  Returns (codes [2F, K/2], scales
    [2F, K/16]); the global scales stay the projections' own (pass them as {gate, up})."""
    _require_operand(gate, "gate")
    _require_operand(up, "up")
    F, K = gate.rows, gate.cols
    _require(up.rows == F and up.cols == K, "gate and up must have the same shape")
    dev = gate.codes.device
    _require(up.codes.device == dev, "gate and up must be on one device")
    w_codes = torch.empty((2 * F, K // 2), dtype=torch.uint8, device=dev)
    w_scales = torch.empty((2 * F, K // 16), dtype=torch.uint8, device=dev)
    _on_gpu(dev)
    st = lib.nvfp4_interleave_gate_up(F, K, _ptr(gate.codes), _ptr(gate.scales), _ptr(up.codes), _ptr(up.scales),
                                      _ptr(w_codes), _ptr(w_scales), _stream(dev))
    _check(st, "nvfp4_interleave_gate_up")
    return w_codes, w_scales


def gemm_swiglu(a: NVFP4Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, w_globals: torch.Tensor,
                h_dtype: torch.dtype | None = torch.bfloat16, h_global: torch.Tensor | None = None,
                out: torch.Tensor | None = None,
                q_out: NVFP4Tensor | None = None) -> tuple[torch.Tensor | None, NVFP4Tensor | None]:
    """Gated MLP input projection in one launch: h = silu(A . Wg^T) * (A . Wu^T) with the
    weights in interleave_gate_up's layout and w_globals = fp32 GPU tensor [2] = {gate, up}.
    h is returned as h_dtype [M, F] unless h_dtype is None, and as NVFP4 under the given
    h_global (fp32 GPU tensor of one element) when h_global is set.  Returns (h, h_nvfp4)."""
    _require(isinstance(w_codes, torch.Tensor) and w_codes.dim() == 2 and w_codes.shape[0] % 32 == 0,
             "w_codes: [2F, K/2], F a multiple of 16")
    F = w_codes.shape[0] // 2
    M, K, _, dev = _fused_weight_checks(a, w_codes, w_scales, (F, F), w_globals)
    _require(h_dtype is not None or h_global is not None, "ask for h, its NVFP4 encoding, or both")
    h = _out_tensor(M, F, h_dtype, dev, out) if h_dtype is not None else None
    q = None
    if h_global is not None:
        _require_f32(h_global, 1, "h_global", dev)
        q = q_out if q_out is not None else NVFP4Tensor(
            torch.empty((M, F // 2), dtype=torch.uint8, device=dev),
            torch.empty((M, F // 16), dtype=torch.uint8, device=dev), h_global)
        _require_bytes(q.codes, (M, F // 2), "q_out.codes", dev)
        _require_bytes(q.scales, (M, F // 16), "q_out.scales", dev)
        q.global_scale = h_global
    per_row = _a_global_per_row(a)
    _on_gpu(dev)
    st = lib.nvfp4_gemm_swiglu(M, F, K, _ptr(a.codes), _ptr(a.scales), _ptr(a.global_scale), per_row,
                               _ptr(w_codes), _ptr(w_scales), _ptr(w_globals), _ptr(h),
                               _y_dtype(h_dtype) if h is not None else _BF16,
                               h.stride(0) if h is not None and M > 0 else F, _ptr(h_global),
                               _ptr(q.codes) if q else None, _ptr(q.scales) if q else None, _stream(dev))
    _check(st, "nvfp4_gemm_swiglu")
    return h, q


def fp8_kv_quantize(x: torch.Tensor, scale: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """FP8 (E4M3FN) bytes of a contiguous bf16/fp32 GPU tensor under the calibrated scale
    (fp32 GPU tensor of one element); the result has x's shape, dtype uint8."""
    _require(x.is_contiguous() and x.dtype in (torch.bfloat16, torch.float32), "x: contiguous bf16/fp32")
    _require_f32(scale, 1, "scale", x.device)
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    _require_bytes(q, tuple(x.shape), "out", x.device)
    _on_gpu(x.device)
    st = lib.nvfp4_fp8_kv_quantize(_ptr(x), _BF16 if x.dtype == torch.bfloat16 else _F32, x.numel(), _ptr(scale),
                                   _ptr(q), _stream(x.device))
    _check(st, "nvfp4_fp8_kv_quantize")
    return q


def fp8_kv_dequantize(q: torch.Tensor, scale: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """Values fl32(E4M3(q) * scale) of FP8 bytes, as bf16 or fp32 (same shape as q)."""
    _require_bytes(q, tuple(q.shape), "q", q.device)
    _require_f32(scale, 1, "scale", q.device)
    y = torch.empty(q.shape, dtype=out_dtype, device=q.device) if out is None else out
    _require(y.device == q.device, "out: a tensor on q's device")
    _require(y.shape == q.shape and y.dtype == out_dtype and y.is_contiguous(), "bad out tensor")
    _on_gpu(q.device)
    st = lib.nvfp4_fp8_kv_dequantize(_ptr(q), q.numel(), _ptr(scale), _ptr(y), _y_dtype(out_dtype), _stream(q.device))
    _check(st, "nvfp4_fp8_kv_dequantize")
    return y
