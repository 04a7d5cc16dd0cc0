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


def gate_bounds(Y: np.ndarray, T: np.ndarray, H: int, a_log, dt_bias, g_o: np.ndarray, beta_o: np.ndarray):
    """Allowed |error| of the kernel's (g, beta) against the oracle's, derived from the
    arithmetic: the kernel's fp32 pre-activation y is within e = 1e-4 * T of the exact one (the
    GEMM bound), which moves each gate by at most the function's largest slope on [y - e, y + e]
    times e (for the decay, plus the fp32 rounding of z = y + dt_bias); the fp32 evaluation of
    exp, log1p, the division and the products adds a few ulps (2e-6 relative); results below
    the fp32 normal range (2^-126) are absolute."""
    N = Y.shape[1]
    yb, ya = Y[:, N - 2 * H:N - H], Y[:, N - H:]
    eb, ea = 1e-4 * T[:, N - 2 * H:N - H], 1e-4 * T[:, N - H:]
    near0 = np.where(np.abs(yb) <= eb, 0.0, np.abs(yb) - eb)     # the point nearest 0
    slope = ref.sigmoid(near0) * ref.sigmoid(-near0)               # s (1 - s), without cancellation
    bound_beta = slope * eb + 2e-6 * np.abs(beta_o) + 2.0 ** -126
    al = np.asarray(a_log, np.float32).astype(np.float64)[None, :]
    z = ya + np.asarray(dt_bias, np.float32).astype(np.float64)[None, :]
    ez = ea + 2.0 ** -23 * np.abs(z)
    bound_g = np.exp(al) * ref.sigmoid(z + ez) * ez + 2e-6 * np.abs(g_o) + np.exp(al) * 2.0 ** -126
    return bound_g, bound_beta


def assert_gates_close(g: torch.Tensor, beta: torch.Tensor, Y: np.ndarray, T: np.ndarray, H: int, a_log, dt_bias,
                       g_o: np.ndarray, beta_o: np.ndarray, what: str = "") -> None:
    bg, bb = gate_bounds(Y, T, H, a_log, dt_bias, g_o, beta_o)
    gh = g.cpu().numpy().astype(np.float64)
    bh = beta.cpu().numpy().astype(np.float64)
    for name, got, want, bound in (("g", gh, g_o, bg), ("beta", bh, beta_o, bb)):
        err = np.abs(got - want)
        bad = np.argwhere(~(err <= bound))
        assert bad.size == 0, (f"{what} {name}: {len(bad)} out of tolerance, first {bad[:3].tolist()} "
                               f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")


def swiglu_bound(H, yg, tg, yu, tu, h: torch.Tensor) -> np.ndarray:
    """Allowed |h - H| for the SwiGLU epilogue: the GEMM bound 1e-4 * T of each product moved
    through silu (slope at most 1.1 in magnitude) and the product, plus (|y_gate| + 4) 2^-23 of
    H for the fp32 evaluation (hardware exponential and reciprocal within one ulp each, on an
    argument rounded to fp32), plus 1e-30 (silu of y < -88 flushes to -0), plus half a bf16 ulp
    for bf16 h."""
    eg, eu = 1e-4 * tg, 1e-4 * tu
    b = 1.1 * eg * (np.abs(yu) + eu) + np.abs(ref.silu(yg)) * eu + (np.abs(yg) + 4.0) * 2.0**-23 * np.abs(H) + 1e-30
    if h.dtype == torch.bfloat16:
        hh = h.float().cpu().numpy().astype(np.float64)
        b = b + half_ulp_bf16(np.maximum(np.abs(hh), np.abs(H)))
    return b


def assert_swiglu_close(h: torch.Tensor, H, yg, tg, yu, tu, what: str = "") -> float:
    hh = h.float().cpu().numpy().astype(np.float64)
    err = np.abs(hh - H)
    bound = swiglu_bound(H, yg, tg, yu, tu, h)
    bad = np.argwhere(~(err <= bound))
    worst = float(np.max(err / bound))
    assert bad.size == 0, (f"{what}: {len(bad)} of {H.size} values out of tolerance, first {bad[:3].tolist()}, "
                           f"max err/bound {worst:.3g}")
    return worst
