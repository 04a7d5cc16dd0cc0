"""Pins for the oracle's E2M1 and E4M3 element formats, against things other than the
oracle itself: the bit-level definitions, an exact rational nearest search, a second
rounding algorithm (per-binade quantum with numpy.rint), and torch's float8_e4m3fn."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref


def _e2m1_from_bits(c: int) -> float:
    """E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is subnormal (m/2)."""
    s, e, m = c >> 3, (c >> 1) & 3, c & 1
    mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
    return -mag if s else mag


def _e4m3_from_bits(b: int) -> Fraction:
    """E4M3FN (OCP): 1 sign, 4 exponent (bias 7), 3 mantissa; exponent 0 subnormal."""
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    mag = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
    return -mag if s else mag


# ---------------------------------------------------------------- E2M1

def test_e2m1_value_set():
    # The sixteen codes give exactly {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}.
    vals = ref.e2m1_decode(np.arange(16))
    assert sorted(set(np.abs(vals).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        assert vals[c] == _e2m1_from_bits(c)
        assert math.copysign(1.0, vals[c]) == (-1.0 if c & 8 else 1.0)


def _e2m1_quantum_rne(v: np.ndarray) -> np.ndarray:
    """Independent algorithm: round to the E2M1 grid spacing of v's binade with numpy.rint
    (round half to even), then saturate at 6, then map the value to its index."""
    v = v.astype(np.float64)
    q = np.where(v < 2.0, 0.5, np.where(v < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(v / q) * q, 6.0)
    lut = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    return np.vectorize(lut.__getitem__, otypes=[np.int64])(r)


def test_e2m1_rne_exhaustive_0p125_to_8():
    # Every float32 from 0.125 to 8.0 (all rounding boundaries of E2M1 lie in this range).
    lo = np.float32(0.125).view(np.uint32)
    hi = np.float32(8.0).view(np.uint32)
    step = 1 << 21
    for start in range(int(lo), int(hi) + 1, step):
        bits = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        v = bits.view(np.float32)
        got = ref.e2m1_rne_sat(v)
        v64 = v.astype(np.float64)
        q = np.where(v64 < 2.0, 0.5, np.where(v64 < 4.0, 1.0, 2.0))
        r = np.minimum(np.rint(v64 / q) * q, 6.0)
        want = np.searchsorted(ref.E2M1_MAGNITUDES, r)   # r is on the grid: exact position
        assert np.array_equal(got, want), f"mismatch in chunk starting at {start:#x}"


def test_e2m1_rne_outside_window():
    g = np.random.default_rng(5)
    small = g.integers(0, np.float32(0.125).view(np.uint32), 200_000, dtype=np.uint32).view(np.float32)
    big = g.integers(np.float32(8.0).view(np.uint32), np.float32(np.inf).view(np.uint32) + 1,
                     200_000, dtype=np.uint32).view(np.float32)
    assert (ref.e2m1_rne_sat(small) == 0).all()
    assert (ref.e2m1_rne_sat(big) == 7).all()
    assert ref.e2m1_rne_sat(np.float32(np.inf)) == 7
    assert np.array_equal(ref.e2m1_rne_sat(small[:1000]), _e2m1_quantum_rne(small[:1000]))


def test_e2m1_rne_exact_rational():
    # Exact nearest search with Fractions, ties to the even index, on values around every
    # midpoint and grid point (+-40 ulps) and random values.
    grid = [Fraction(x).limit_denominator(4) for x in ref.E2M1_MAGNITUDES]
    pts = []
    for a, b in zip(ref.E2M1_MAGNITUDES[:-1], ref.E2M1_MAGNITUDES[1:]):
        for c in (a, (a + b) / 2):
            u = np.float32(c).view(np.uint32)
            pts.extend(np.arange(max(int(u) - 40, 0), int(u) + 41, dtype=np.uint32).view(np.float32))
    pts.extend(np.random.default_rng(1).uniform(0, 7, 3000).astype(np.float32))
    pts = np.array(pts, dtype=np.float32)
    got = ref.e2m1_rne_sat(pts)
    for v, gi in zip(pts.tolist(), got.tolist()):
        fv = Fraction(v)
        d = [abs(fv - g) for g in grid]
        best = min(d)
        cand = [i for i, di in enumerate(d) if di == best]
        want = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
        assert gi == want, (v, gi, want)


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_all_bytes_vs_torch():
    b = torch.arange(256, dtype=torch.uint8)
    t = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    o = ref.e4m3_decode(np.arange(256))
    nan_t, nan_o = np.isnan(t), np.isnan(o)
    assert np.array_equal(nan_t, nan_o)
    assert nan_o.sum() == 2 and nan_o[0x7F] and nan_o[0xFF]
    assert np.array_equal(t[~nan_t], o[~nan_o])
    for byte in range(256):
        if byte & 0x7F != 0x7F:
            assert Fraction(o[byte]) == _e4m3_from_bits(byte)
    assert o[0x7E] == 448.0 and o[0x38] == 1.0 and o[0x01] == 2.0 ** -9 and o[0x08] == 2.0 ** -6


def test_e4m3_table_monotone():
    assert ref.E4M3_TABLE.size == 127
    assert np.all(np.diff(ref.E4M3_TABLE) > 0)


def _near_boundaries_e4m3(width: int) -> np.ndarray:
    vals = ref.E4M3_TABLE
    mids = (vals[:-1] + vals[1:]) / 2
    pts = []
    for c in np.concatenate([vals, mids]):
        u = int(np.float32(c).view(np.uint32))
        pts.append(np.arange(max(u - width, 0), u + width + 1, dtype=np.uint32))
    return np.concatenate(pts).view(np.float32)


def test_e4m3_rne_vs_torch():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even and saturates up to 464
    # (above that it gives NaN; our encoder saturates to 448 there, tested separately).
    g = np.random.default_rng(7)
    top = int(np.float32(464.0).view(np.uint32))
    rand = g.integers(0, top + 1, 4_000_000, dtype=np.uint32).view(np.float32)
    pts = np.concatenate([rand, _near_boundaries_e4m3(300)])
    pts = pts[pts <= 464.0]
    want = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = ref.e4m3_rne_sat(pts)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(pts[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def test_e4m3_rne_saturates_above_464():
    x = np.array([464.0, 464.00003, 480.0, 1e30, np.inf], dtype=np.float32)
    assert (ref.e4m3_rne_sat(x) == 0x7E).all()


def test_e4m3_rne_exact_rational():
    grid = [_e4m3_from_bits(b) for b in range(0x7F)]
    pts = _near_boundaries_e4m3(3)
    pts = pts[(pts <= 448.0)]
    got = ref.e4m3_rne_sat(pts)
    for v, gb in zip(pts.tolist(), got.tolist()):
        fv = Fraction(v)
        d = [abs(fv - g) for g in grid]
        best = min(d)
        cand = [i for i, di in enumerate(d) if di == best]
        want = cand[0] if len(cand) == 1 else [i for i in cand if i % 2 == 0][0]
        assert gb == want, (v, gb, want)


# ---------------------------------------------------------------- arithmetic environment

def test_float32_denormals_are_kept():
    # The encoder's arithmetic is IEEE binary32 without flush-to-zero.
    tiny = np.float32(1e-40)
    assert tiny * np.float32(0.5) != 0
    assert (np.array([1e-40], np.float32) / np.float32(3.0))[0] != 0


@pytest.mark.parametrize("code", range(16))
def test_dequant_products_exact_in_fp16_and_bf16(code):
    # E2M1 x E4M3 has at most 6 significant bits and lies in [2^-10, 2688]: both half and
    # bfloat16 represent every such product exactly (float8 does not).
    v = ref.e2m1_decode(code)
    prod = v * ref.E4M3_TABLE                       # exact in float64
    for dt in (torch.float16, torch.bfloat16):
        back = torch.from_numpy(prod).to(dt).to(torch.float64).numpy()
        assert np.array_equal(back, prod)
