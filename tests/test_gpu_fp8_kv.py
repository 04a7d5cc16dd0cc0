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
