"""Pins of the oracle's FP8 (E4M3FN) KV-cache codec against what fixes it independently of
the oracle: torch's float8_e4m3fn cast (round to nearest even, a separate implementation)
applied to the IEEE binary32 quotient, exact power-of-two scaling, the saturation and NaN
readings, a round-trip error bound, and torch's float8 decode of all 256 bytes."""
import numpy as np
import torch

from oracle import nvfp4_ref as ref


def _torch_fp8(t32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(t32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def _near_midpoints() -> np.ndarray:
    vals = ref.E4M3_TABLE[np.isfinite(ref.E4M3_TABLE)]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    bits = mids.view(np.uint32).astype(np.int64)
    near = np.concatenate([bits + k for k in range(-3, 4)])
    out = near.astype(np.uint32).view(np.float32)
    out = out[np.abs(out) <= 448.0]
    return np.concatenate([out, -out, vals.astype(np.float32), -vals.astype(np.float32)])


def test_unit_scale_matches_torch_cast_near_every_midpoint():
    t = _near_midpoints()
    assert np.array_equal(ref.fp8_kv_quantize(t, 1.0), _torch_fp8(t))


def test_general_scale_matches_torch_cast_of_ieee_quotient():
    g = np.random.default_rng(5)
    x = (g.standard_normal(200_000) * g.choice([1e-3, 0.1, 1.0, 30.0], 200_000)).astype(np.float32)
    for s in (0.0173, 1.0 / 3.0, 0.75, 2.5e-3):
        q = torch.from_numpy(x) / torch.tensor(np.float32(s))       # IEEE binary32 division
        t = q.numpy()
        keep = np.abs(t) <= 448.0                                    # torch's cast does not saturate
        assert np.array_equal(ref.fp8_kv_quantize(x, s)[keep], _torch_fp8(t[keep])), s


def test_power_of_two_scale_is_an_exact_shift():
    # Dividing by 2^k is exact, so the scale must act as a divisor: q(x, 2^k) == q(x / 2^k, 1).
    t = _near_midpoints()
    for k in (-5, 3, 9):
        assert np.array_equal(ref.fp8_kv_quantize(t * np.float32(2.0 ** k), 2.0 ** k), ref.fp8_kv_quantize(t, 1.0))


def test_saturation_nan_and_signed_zero():
    x = np.array([448.0, 463.9, 464.0, 1e30, np.inf, -500.0, -np.inf, np.nan, -0.0, 0.0], np.float32)
    got = ref.fp8_kv_quantize(x, 1.0)
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x00]


def test_round_trip_error_bound():
    g = np.random.default_rng(6)
    s = np.float32(0.0371)
    x = (g.uniform(-448, 448, 100_000) * s).astype(np.float32)
    y = ref.fp8_kv_dequantize(ref.fp8_kv_quantize(x, s), s).astype(np.float64)
    err = np.abs(y - x)
    assert np.all(err <= 2.0 ** -4 * np.abs(x) * (1 + 1e-6) + 2.0 ** -10 * s)


def test_dequantize_every_byte_matches_torch_decode():
    b = np.arange(256, dtype=np.uint8)
    s = np.float32(0.0371)
    want = (torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(s)).numpy()
    got = ref.fp8_kv_dequantize(b, s)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin]) and np.all(np.isnan(got[~fin]))
