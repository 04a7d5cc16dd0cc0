"""GPU parity of the FP8 (E4M3FN) KV-cache codec against the oracle: quantized bytes bit for
bit, dequantized fp32 values bit for bit (NaN where the oracle has NaN), and bf16 output
equal to the round-to-nearest-even bf16 of the oracle's fp32 values.  Inputs mix random
values over the whole E4M3 range, exact rounding ties, saturating and special values, and
lengths whose last n % 8 elements take the elementwise tail."""
import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, nv

pytestmark = pytest.mark.gpu


def _inputs(n, s, seed):
    g = np.random.default_rng(seed)
    x = (g.standard_normal(n) * g.choice([1e-4, 0.01, 1.0, 50.0], n)).astype(np.float32) * np.float32(s) * 40
    vals = ref.E4M3_TABLE[np.isfinite(ref.E4M3_TABLE)]
    mids = ((vals[1:] + vals[:-1]) / 2) * s                       # ties (up to fp32 rounding of the product)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 448 * s, 464 * s, -500 * s, 1e30, -1e-30,
                        2.0 ** -10 * s, 1.5 * 2.0 ** -10 * s], np.float32)
    k = min(n, len(mids) + len(special))
    fill = np.concatenate([mids.astype(np.float32), special])[:k]
    x[g.choice(n, k, replace=False)] = fill
    return x


@pytest.mark.parametrize("n", [1, 7, 8, 4099, 1_000_003])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("s", [0.0371, 2.0 ** -5, 1.0 / 3.0])
def test_quantize_dequantize_bitwise(n, dtype, s):
    x = _inputs(n, s, seed=n)
    xg = torch.from_numpy(x).to(DEV).to(dtype)
    x_in = xg.float().cpu().numpy()                              # the values the kernel reads
    sg = torch.tensor([s], dtype=torch.float32, device=DEV)
    q = nv().fp8_kv_quantize(xg, sg)
    want = ref.fp8_kv_quantize(x_in, np.float32(s))
    got = q.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first {[(int(i), x_in[i], got[i], want[i]) for i in bad[:3, 0]]}"
    y32 = nv().fp8_kv_dequantize(q, sg, torch.float32).cpu().numpy()
    w32 = ref.fp8_kv_dequantize(want, np.float32(s))
    nan = np.isnan(w32)
    assert np.array_equal(np.isnan(y32), nan)
    assert np.array_equal(y32[~nan].view(np.uint32), w32[~nan].view(np.uint32))
    y16 = nv().fp8_kv_dequantize(q, sg, torch.bfloat16).cpu()
    w16 = torch.from_numpy(w32).to(torch.bfloat16)
    assert torch.equal(torch.isnan(y16), torch.isnan(w16))
    ok = ~torch.isnan(w16)
    assert torch.equal(y16[ok].view(torch.int16), w16[ok].view(torch.int16))


def test_kv_cache_shaped_tensor_round_trip():
    # A K cache of 8192 tokens x 8 heads x 128 dims under its calibrated scale max|K| / 448.
    g = torch.Generator(device="cpu").manual_seed(11)
    k = (torch.randn(8192, 8, 128, generator=g) * torch.linspace(0.2, 3.0, 128)).to(torch.bfloat16)
    kg = k.to(DEV)
    s = np.float32(float(k.float().abs().max()) / 448.0)
    sg = torch.tensor([s], dtype=torch.float32, device=DEV)
    q = nv().fp8_kv_quantize(kg, sg)
    assert q.shape == k.shape
    want = ref.fp8_kv_quantize(k.float().numpy().reshape(-1), s)
    assert np.array_equal(q.cpu().numpy().reshape(-1), want)
    back = nv().fp8_kv_dequantize(q, sg, torch.float32).cpu().numpy().reshape(-1)
    x = k.float().numpy().reshape(-1)
    assert np.all(np.abs(back - x) <= 2.0 ** -4 * np.abs(x) * (1 + 1e-6) + 2.0 ** -10 * s)


def test_empty():
    sg = torch.tensor([1.0], dtype=torch.float32, device=DEV)
    assert nv().fp8_kv_quantize(torch.empty(0, dtype=torch.bfloat16, device=DEV), sg).numel() == 0


# Scales inside the quantizer's fast range [2^-64, 2^64] (its edges included) and outside it.
FAST_SCALES = [1.0, 0.0371, 1.0 / 3.0, 2.0 ** -64, 2.0 ** 64, 3.0e-19, 7.7e17]
SLOW_SCALES = [2.0 ** -64 * 0.75, 2.0 ** 64 * 1.5, 2.0 ** -70, 2.0 ** 70, 1e-40]


def _bitwise_quantize(x32: np.ndarray, dtype, s: float, what: str) -> None:
    xg = torch.from_numpy(x32).to(DEV).to(dtype)
    sg = torch.tensor([s], dtype=torch.float32, device=DEV)
    got = nv().fp8_kv_quantize(xg, sg).cpu().numpy()
    want = ref.fp8_kv_quantize(xg.float().cpu().numpy(), np.float32(s))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{what} s={s!r}: {bad.size} bytes differ, first "
                           f"{[(float(x32[i]), int(got[i]), int(want[i])) for i in bad[:3]]}")


@pytest.mark.parametrize("order", ["sorted", "shuffled_no_nan"])
@pytest.mark.parametrize("s", FAST_SCALES + SLOW_SCALES)
def test_every_bf16_value(s, order):
    """All 65536 bf16 bit patterns.  In bit order the NaN patterns sit together, so nearly
    every wave takes the fast path; shuffled (NaNs left out) every wave does."""
    x = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    if order == "shuffled_no_nan":
        x = x[~np.isnan(x)]
        x = x[np.random.default_rng(5).permutation(x.size)]
    _bitwise_quantize(x, torch.bfloat16, s, order)


def _decision_neighbourhoods(s: float, ulps: int = 8) -> np.ndarray:
    """fp32 dividends within +-ulps of fl32(t s) for every E4M3 decision point t (midpoints
    of neighbouring values), the clamp and saturation region and the zero boundary, both
    signs."""
    vals = ref.E4M3_TABLE[np.isfinite(ref.E4M3_TABLE)].astype(np.float64)
    t = np.concatenate([(vals[1:] + vals[:-1]) / 2, [440.0, 448.0, 464.0, 1024.0, 2.0 ** 20, 2.0 ** -12]])
    c = (t * np.float64(np.float32(s))).astype(np.float32)
    c = c[np.isfinite(c) & (c > 0)]
    k = np.arange(-ulps, ulps + 1, dtype=np.int64)
    bits = (c.view(np.uint32).astype(np.int64)[:, None] + k[None, :]).reshape(-1)
    x = bits[(bits > 0) & (bits < 0x7F800000)].astype(np.uint32).view(np.float32)
    return np.concatenate([x, -x])


@pytest.mark.parametrize("s", FAST_SCALES + SLOW_SCALES)
def test_fp32_near_every_decision_point(s):
    _bitwise_quantize(_decision_neighbourhoods(s), torch.float32, s, "decision points")


def test_fp32_decision_points_over_random_scales():
    """Sixty-four scales log-uniform over the fast range and past both of its ends."""
    g = np.random.default_rng(17)
    scales = np.exp2(g.uniform(-70.0, 70.0, 64)).astype(np.float32)
    x = np.concatenate([_decision_neighbourhoods(float(s), ulps=3) for s in scales])
    for s in scales:                                   # every scale on every dividend set
        _bitwise_quantize(x, torch.float32, float(s), "random scales")


def test_fp32_random_values_across_the_range():
    """2M fp32 values with exponents uniform over the whole binary32 range, plus infinities,
    NaNs and signed zeros scattered through them."""
    g = np.random.default_rng(23)
    bits = (g.integers(0, 255, 2_000_000, dtype=np.uint32) << 23) | g.integers(0, 1 << 23, 2_000_000, dtype=np.uint32)
    bits |= g.integers(0, 2, 2_000_000, dtype=np.uint32) << 31
    x = bits.view(np.float32).copy()
    x[g.choice(x.size, 64, replace=False)] = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-45, -1e-45, 3e38] * 8,
                                                      np.float32)
    for s in (1.0, 2.0 ** -40, 2.0 ** 40, 2.0 ** -70):
        _bitwise_quantize(x, torch.float32, s, "random")


@pytest.mark.parametrize("s", [1.0, 0.0371, 2.0 ** -64, 2.0 ** 70, 1e-40])
def test_dequantize_every_byte(s):
    q = np.tile(np.arange(256, dtype=np.uint8), 9)[: 256 * 9 - 3]        # ragged: elementwise tail too
    sg = torch.tensor([s], dtype=torch.float32, device=DEV)
    qg = torch.from_numpy(q).to(DEV)
    w32 = ref.fp8_kv_dequantize(q, np.float32(s))
    y32 = nv().fp8_kv_dequantize(qg, sg, torch.float32).cpu().numpy()
    nan = np.isnan(w32)
    assert np.array_equal(np.isnan(y32), nan)
    assert np.array_equal(y32[~nan].view(np.uint32), w32[~nan].view(np.uint32))
    y16 = nv().fp8_kv_dequantize(qg, sg, torch.bfloat16).cpu()
    w16 = torch.from_numpy(w32).to(torch.bfloat16)
    assert torch.equal(torch.isnan(y16), torch.isnan(w16))
    ok = ~torch.isnan(w16)
    assert torch.equal(y16[ok].view(torch.int16), w16[ok].view(torch.int16))
