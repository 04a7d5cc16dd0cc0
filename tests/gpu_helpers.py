"""Helpers for the GPU parity tests: move seeded inputs and oracle tensors to the GPU and
compare the library's outputs with the oracle.

The HIP binding is imported lazily (``nv()``) so that CPU-only test collection does not
need it; on a machine with a GPU a missing library makes every GPU test fail loudly."""
from __future__ import annotations

import numpy as np
import torch

from oracle import nvfp4_ref as ref

DEV = torch.device("cuda:0")


def nv():
    import nvfp4_w4a4_block_amd as m
    return m


def to_gpu(x: np.ndarray, bf16: bool = True) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def to_host(q) -> ref.NVFP4:
    """Library NVFP4Tensor -> oracle NVFP4 (numpy)."""
    return ref.NVFP4(q.codes.cpu().numpy(), q.scales.cpu().numpy(),
                     q.global_scale.float().cpu().numpy(), q.rows, q.cols)


def to_device(q: ref.NVFP4):
    return nv().NVFP4Tensor(torch.from_numpy(q.codes).to(DEV), torch.from_numpy(q.scales).to(DEV),
                            torch.from_numpy(np.asarray(q.global_scale, np.float32)).to(DEV))


def assert_quant_equal(got, want: ref.NVFP4, rows=None, what: str = "") -> None:
    """Bit-exact comparison of codes, scale bytes and global scales."""
    g = to_host(got) if not isinstance(got, ref.NVFP4) else got
    gc, gs = g.codes, g.scales
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert gc.shape == want.codes.shape and gs.shape == want.scales.shape, what
    gg = np.asarray(g.global_scale, np.float32).view(np.uint32)
    wg = np.asarray(want.global_scale, np.float32).view(np.uint32)
    if rows is None:
        assert np.array_equal(gg, wg), f"{what}: global scale {g.global_scale} vs {want.global_scale}"
    bad = np.argwhere(gs != want.scales)
    assert bad.size == 0, f"{what}: {len(bad)} scale bytes differ, first {bad[:3].tolist()}"
    bad = np.argwhere(gc != want.codes)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first {bad[:3].tolist()}"


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |v| (normal range)."""
    _, e = np.frexp(np.abs(v))
    return np.ldexp(1.0, e - 9)


def gemm_errors(y: torch.Tensor, Y: np.ndarray, T: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-element |y - Y| and the allowed bound: 1e-4 * T, plus half a bf16 ulp of
    max(|y|, |Y|) when y is bf16."""
    yh = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(yh - Y)
    bound = 1e-4 * T
    if y.dtype == torch.bfloat16:
        bound = bound + half_ulp_bf16(np.maximum(np.abs(yh), np.abs(Y)))
    return err, bound


def assert_gemm_close(y: torch.Tensor, Y: np.ndarray, T: np.ndarray, what: str = "") -> float:
    err, bound = gemm_errors(y, Y, T)
    bad = np.argwhere(~(err <= bound))
    worst = float(np.max(err / np.maximum(T, 1e-300)))
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first {bad[:3].tolist()}, "
                           f"max err/T {worst:.3g}")
    return worst
