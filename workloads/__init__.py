"""Seeded synthetic inputs for the NVFP4 W4A4 hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests, ``bench.py`` and
``__graft_entry__.smoke``.  It holds shapes and random draws only: no NVFP4 arithmetic
(no scales, no rounding to E2M1/E4M3, no GEMM).  The one numeric step here is rounding the
float32 draws to bfloat16-representable values, because the activations and weights of the
served model are bf16 tensors; the method starts from those bf16 values.

The workloads stand in for the ones the pages describe: the residual-stream activations of
a 64-layer hybrid model (48 Gated DeltaNet + 16 attention layers, hidden 5120, MLP 17408)
with hot channels far above the median ("Why Gated DeltaNet Survives 4-Bit Quantization"
page, "The deep dive": outlier channels about a hundred times the median, 496 linears), and
its linear-layer weights.  The trained checkpoint and the evaluation data are not available,
so every tensor is a seeded Gaussian draw of the right shape with planted outlier channels.

Generator: ``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id])))``,
``standard_normal(dtype=float32) * sigma``, outlier channels multiplied afterwards, then
round-to-nearest-even to bf16 (for bf16 workloads).  Outlier channels are
``round(frac * K)`` distinct input channels drawn with ``Generator.choice`` from the same
generator after the Gaussian draw.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng",
    "round_to_bf16",
    "activation",
    "weight",
    "TINY",
    "PREFILL",
    "DECODE",
    "DECODE_UP",
    "FUSED",
    "MLP",
    "SWEEP",
    "sweep_launches",
    "Launch",
]


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    """Counter-free, reproducible generator for tensor ``tensor_id`` of workload ``seed``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Non-finite values are passed through unchanged (NaN stays NaN).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    r = np.where(np.isfinite(x), r, u).astype(np.uint32)
    return r.view(np.float32)


def _outlier_channels(g: np.random.Generator, k: int, frac: float | None,
                      explicit: tuple[int, ...] | None) -> np.ndarray:
    if explicit is not None:
        return np.asarray(explicit, dtype=np.int64)
    if not frac:
        return np.zeros(0, dtype=np.int64)
    n = int(round(frac * k))
    return np.sort(g.choice(k, size=n, replace=False)).astype(np.int64)


def activation(seed: int, tensor_id: int, rows: int, cols: int, *, sigma: float = 1.0,
               outlier_frac: float | None = None, outlier_channels: tuple[int, ...] | None = None,
               outlier_gain: float = 50.0, bf16: bool = True) -> np.ndarray:
    """Activations X[rows, cols] ~ N(0, sigma^2) with hot input channels (columns).

    Returns float32; when ``bf16`` the values are exactly representable in bfloat16.
    """
    g = rng(seed, tensor_id)
    x = g.standard_normal((rows, cols), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    ch = _outlier_channels(g, cols, outlier_frac, outlier_channels)
    if ch.size:
        x[:, ch] *= np.float32(outlier_gain)
    return round_to_bf16(x) if bf16 else x


def weight(seed: int, tensor_id: int, rows: int, cols: int, *, sigma: float = 0.02,
           bf16: bool = True) -> np.ndarray:
    """Weights W[rows=N, cols=K] ~ N(0, sigma^2), K-major like the activations."""
    g = rng(seed, tensor_id)
    w = g.standard_normal((rows, cols), dtype=np.float32)
    w *= np.float32(sigma)
    return round_to_bf16(w) if bf16 else w


# ---------------------------------------------------------------------------------------
# The five workloads.  Shapes follow the hybrid model the pages describe (hidden 5120,
# MLP 17408, 48 GDN + 16 attention layers); tensor ids are fixed so every consumer
# draws identical tensors.
# ---------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Tiny:
    """16x256 fp32 activations with channels 3 and 97 scaled x40; 128x256 fp32 weights."""
    name: str = "tiny"
    seed: int = 0
    M: int = 16
    N: int = 128
    K: int = 256
    outlier_channels: tuple[int, ...] = (3, 97)
    outlier_gain: float = 40.0
    w_sigma: float = 0.02

    def x(self) -> np.ndarray:
        return activation(self.seed, 0, self.M, self.K, outlier_channels=self.outlier_channels,
                          outlier_gain=self.outlier_gain, bf16=False)

    def w(self) -> np.ndarray:
        return weight(self.seed, 1, self.N, self.K, sigma=self.w_sigma, bf16=False)


@dataclass(frozen=True)
class Prefill:
    """Prefill up-projection: X[4096x5120] bf16, 0.1% channels x50; W[17408x5120] bf16."""
    name: str = "prefill"
    seed: int = 1
    M: int = 4096
    N: int = 17408
    K: int = 5120
    outlier_frac: float = 0.001
    outlier_gain: float = 50.0
    w_sigma: float = 0.02

    def x(self, rows: int | None = None) -> np.ndarray:
        return activation(self.seed, 0, rows or self.M, self.K, outlier_frac=self.outlier_frac,
                          outlier_gain=self.outlier_gain)

    def w(self) -> np.ndarray:
        return weight(self.seed, 1, self.N, self.K, sigma=self.w_sigma)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


@dataclass(frozen=True)
class Decode:
    """Decode down-projection: X[M x 17408] bf16 with M in {1,4,16}; W[5120x17408].  The same
    class with N and K swapped is the MLP up projection at decode."""
    name: str = "decode"
    seed: int = 2
    Ms: tuple[int, ...] = (1, 4, 16)
    N: int = 5120
    K: int = 17408
    w_sigma: float = 0.02

    def x(self, M: int) -> np.ndarray:
        # One activation tensor per token count, so each M draws its own tokens.
        return activation(self.seed, 100 + M, M, self.K)

    def w(self) -> np.ndarray:
        return weight(self.seed, 1, self.N, self.K, sigma=self.w_sigma)


@dataclass(frozen=True)
class Mlp:
    """Gated MLP input projection: X[M x 5120] bf16 (0.1% channels x50), gate and up weights
    [17408 x 5120] each; prefill M = 4096, decode M in {1, 16}."""
    name: str = "mlp"
    seed: int = 5
    M: int = 4096
    Ms: tuple[int, ...] = (1, 16)
    F: int = 17408
    K: int = 5120
    outlier_frac: float = 0.001
    outlier_gain: float = 50.0
    w_sigma: float = 0.02

    def x(self, rows: int) -> np.ndarray:
        # One activation tensor per token count (ids 100 + rows, clear of the weights' 1, 2).
        return activation(self.seed, 100 + rows, rows, self.K, outlier_frac=self.outlier_frac,
                          outlier_gain=self.outlier_gain)

    def gate(self) -> np.ndarray:
        return weight(self.seed, 1, self.F, self.K, sigma=self.w_sigma)

    def up(self) -> np.ndarray:
        return weight(self.seed, 2, self.F, self.K, sigma=self.w_sigma)


@dataclass(frozen=True)
class Fused:
    """Fused GDN input projections: six modules, each with its own sigma and global scale."""
    name: str = "fused"
    seed: int = 3
    M: int = 8192
    K: int = 5120
    widths: tuple[int, ...] = (2048, 2048, 4096, 4096, 48, 48)
    sigmas: tuple[float, ...] = (0.02, 0.02, 0.015, 0.015, 0.05, 0.05)
    outlier_frac: float = 0.001
    outlier_gain: float = 50.0

    @property
    def N(self) -> int:
        return int(sum(self.widths))

    def x(self, rows: int | None = None) -> np.ndarray:
        return activation(self.seed, 0, rows or self.M, self.K, outlier_frac=self.outlier_frac,
                          outlier_gain=self.outlier_gain)

    def w(self, i: int) -> np.ndarray:
        return weight(self.seed, 1 + i, self.widths[i], self.K, sigma=self.sigmas[i])

    def gate_params(self) -> tuple[np.ndarray, np.ndarray]:
        """Per-head parameters of the two gate segments (one head per column of the last
        two widths): A_log ~ U(0, ln 16) and dt_bias ~ U(-6.9, -2.25), float32.  The pages
        give no trained values; these ranges put the per-step decay of the synthetic heads
        anywhere from nearly none to strong."""
        h = self.widths[-1]
        a_log = rng(self.seed, 100).uniform(0.0, np.log(16.0), h).astype(np.float32)
        dt_bias = rng(self.seed, 101).uniform(-6.9, -2.25, h).astype(np.float32)
        return a_log, dt_bias


@dataclass(frozen=True)
class Launch:
    layer: int
    kind: str            # "gdn_in", "gdn_out", "attn_qkv", "attn_o", "mlp_gate_up", "mlp_down"
    K: int
    widths: tuple[int, ...]

    @property
    def N(self) -> int:
        return int(sum(self.widths))


@dataclass(frozen=True)
class Sweep:
    """All linear GEMMs of a synthetic 64-layer hybrid at M=16384 prefill tokens."""
    name: str = "sweep"
    seed: int = 4
    M: int = 16384
    layers: int = 64
    hidden: int = 5120
    mlp: int = 17408
    gdn_widths: tuple[int, ...] = (2048, 2048, 4096, 4096, 48, 48)
    gdn_value_width: int = 4096
    outlier_frac: float = 0.001
    outlier_gain: float = 50.0
    w_sigma: float = 0.02
    launches: tuple[Launch, ...] = field(default=(), compare=False)

    def is_attention(self, layer: int) -> bool:
        # 3 GDN layers then 1 attention layer, repeated: 48 GDN + 16 attention.
        return layer % 4 == 3

    def x(self, launch_index: int, K: int, rows: int | None = None) -> np.ndarray:
        return activation(self.seed, 10_000 + launch_index, rows or self.M, K,
                          outlier_frac=self.outlier_frac, outlier_gain=self.outlier_gain)

    def w(self, launch_index: int, segment: int, N: int, K: int) -> np.ndarray:
        return weight(self.seed, 20_000 + 64 * launch_index + segment, N, K, sigma=self.w_sigma)


def sweep_launches(sw: Sweep | None = None) -> list[Launch]:
    """The 256 GEMM launches of the sweep: per layer one fused input projection, one output
    projection, one fused MLP gate+up and one MLP down projection (4 x 64 = 256)."""
    sw = sw or SWEEP
    h, f = sw.hidden, sw.mlp
    out: list[Launch] = []
    for layer in range(sw.layers):
        if sw.is_attention(layer):
            out.append(Launch(layer, "attn_qkv", h, (h, h, h)))
            out.append(Launch(layer, "attn_o", h, (h,)))
        else:
            out.append(Launch(layer, "gdn_in", h, sw.gdn_widths))
            out.append(Launch(layer, "gdn_out", sw.gdn_value_width, (h,)))
        out.append(Launch(layer, "mlp_gate_up", h, (f, f)))
        out.append(Launch(layer, "mlp_down", f, (h,)))
    return out


TINY = Tiny()
PREFILL = Prefill()
DECODE = Decode()
DECODE_UP = Decode(name="decode_up", seed=4, N=17408, K=5120)
FUSED = Fused()
MLP = Mlp()
SWEEP = Sweep()
