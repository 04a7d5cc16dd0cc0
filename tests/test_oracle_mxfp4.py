"""Pins of the oracle's lossy NVFP4 -> MXFP4 re-encoding and MXFP4 GEMM against what fixes
them independently of the oracle: hand-derived blocks (a lossless case, the clamp of a block
maximum above 6 * 2^e, a tie to even, a small half-block that vanishes, a zero block), a brute
force nearest search with exact rationals and a shared exponent taken from integer bit
lengths, and the GEMM against exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_ref as ref

ONE = 0x38                      # E4M3 byte of 1.0


def _nv(codes_rc, scales_rb, g=1.0) -> ref.NVFP4:
    codes_rc = np.asarray(codes_rc, np.uint8)
    R, C = codes_rc.shape
    return ref.NVFP4(ref.pack_codes(codes_rc), np.asarray(scales_rb, np.uint8).reshape(R, C // 16),
                     np.asarray([g], np.float32), R, C)


def _mx_values(m: ref.MXFP4) -> np.ndarray:
    return ref.mx_dequantize(m) / float(m.global_scale[0])


def test_e8m0_decode():
    assert ref.e8m0_decode(127) == 1.0 and ref.e8m0_decode(128) == 2.0 and ref.e8m0_decode(120) == 2.0 ** -7
    assert np.isnan(ref.e8m0_decode(0xFF))


def test_lossless_power_of_two_scales():
    # Both halves share the E4M3 scale 2^3 (byte 0x50) and the block holds a 6: the MX scale
    # is 2^3 and every code survives unchanged.
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    codes[:, 5] = 7
    codes[:, 37] = 15
    t = _nv(codes, [[0x50] * 4] * 3)
    assert ref.e4m3_decode(0x50) == 8.0
    m = ref.mxfp4_from_nvfp4(t)
    assert np.array_equal(m.scales, np.full((3, 2), 127 + 3, np.uint8))
    assert np.array_equal(m.codes, t.codes)
    assert np.array_equal(ref.mx_dequantize(m), ref.dequantize(t))


def test_hand_derived_block():
    # One 32-block: first half under scale 1.125 (0x39), second half under 10 (0x52).
    assert ref.e4m3_decode(0x39) == 1.125 and ref.e4m3_decode(0x52) == 10.0
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0] = 7          # 6 * 1.125 = 6.75  (the block max: exponent floor(log2 6.75) - 2 = 0)
    codes[0, 1] = 8 | 5      # -3 * 1.125 = -3.375 -> 3 (nearest), sign kept
    codes[0, 16] = 1         # 0.5 * 10 = 5 -> tie between 4 and 6 -> 4 (even index 6)
    codes[0, 2] = 1          # 0.5 * 1.125 = 0.5625 -> 0.5
    codes[0, 3] = 8          # -0 stays -0 (code 8)
    m = ref.mxfp4_from_nvfp4(_nv(codes, [[0x39, 0x52]]))
    assert m.scales[0, 0] == 127
    got = ref.unpack_codes(m.codes)[0]
    assert got[0] == 7 and got[1] == (8 | 5) and got[16] == 6 and got[2] == 1 and got[3] == 8
    v = _mx_values(m)[0]
    assert v[0] == 6.0 and v[1] == -3.0 and v[16] == 4.0 and v[2] == 0.5


def test_small_half_block_vanishes_and_zero_block():
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 0] = 7                       # 6 under scale 1: exponent 0
    codes[0, 20] = 1                      # 0.5 * 2^-6 under scale 2^-6 (byte 0x08): below 0.25 -> 0
    assert ref.e4m3_decode(0x08) == 2.0 ** -6
    m = ref.mxfp4_from_nvfp4(_nv(codes, [[ONE, 0x08, ONE, ONE]]))
    got = ref.unpack_codes(m.codes)[0]
    assert got[20] == 0
    assert m.scales[0, 1] == 0 and np.all(got[32:] == 0)   # the all-zero second block


def _floor_log2(x: Fraction) -> int:
    n, d = x.numerator, x.denominator       # d is a power of two for these values
    e = n.bit_length() - d.bit_length()
    return e if Fraction(2) ** e <= x else e - 1


def test_brute_force_nearest_with_exact_rationals():
    rng = np.random.default_rng(1)
    R, C = 6, 256
    codes = rng.integers(0, 16, (R, C)).astype(np.uint8)
    scales = rng.integers(0x20, 0x60, (R, C // 16)).astype(np.uint8)     # 2^-3 .. 2^4 range
    t = _nv(codes, scales)
    m = ref.mxfp4_from_nvfp4(t)
    v = ref.e2m1_decode(codes) * np.repeat(ref.e4m3_decode(scales), 16, axis=1)
    mags = [Fraction(x) for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    out = ref.unpack_codes(m.codes)
    for r in range(R):
        for b in range(C // 32):
            blk = [Fraction(float(x)) for x in v[r, 32 * b:32 * b + 32]]
            amax = max(abs(x) for x in blk)
            e = _floor_log2(amax) - 2
            assert int(m.scales[r, b]) == e + 127
            X = Fraction(2) ** e
            for i, x in enumerate(blk):
                q = abs(x) / X
                dist = [abs(q - c) for c in mags]
                best = min(dist)
                idx = [k for k, d in enumerate(dist) if d == best]
                want = 7 if q >= 6 else (idx[0] if len(idx) == 1 else [k for k in idx if k % 2 == 0][0])
                c = int(out[r, 32 * b + i])
                assert c & 7 == want and (c >> 3) == (codes[r, 32 * b + i] >> 3), (r, b, i)


def test_mx_gemm_exact_rationals():
    rng = np.random.default_rng(2)
    M, N, K = 3, 4, 64
    a = ref.MXFP4(ref.pack_codes(rng.integers(0, 16, (M, K)).astype(np.uint8)),
                  rng.integers(120, 135, (M, K // 32)).astype(np.uint8), np.asarray([0.75], np.float32), M, K)
    w = ref.MXFP4(ref.pack_codes(rng.integers(0, 16, (N, K)).astype(np.uint8)),
                  rng.integers(120, 135, (N, K // 32)).astype(np.uint8), np.asarray([1.25], np.float32), N, K)
    Y, T = ref.mx_gemm(a, w)
    mag = [Fraction(x) for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]

    def val(t, r, k):
        c = int(ref.unpack_codes(t.codes)[r, k])
        s = Fraction(2) ** (int(t.scales[r, k // 32]) - 127)
        return (-1 if c & 8 else 1) * mag[c & 7] * s * Fraction(float(t.global_scale[0]))

    for i in range(M):
        for j in range(N):
            exact = sum(val(a, i, k) * val(w, j, k) for k in range(K))
            absum = sum(abs(val(a, i, k) * val(w, j, k)) for k in range(K))
            assert Y[i, j] == float(exact) and T[i, j] == float(absum)


def test_reencode_error_is_bounded():
    # Every re-encoded value is within one MX quantum of its NVFP4 value (two for the clamped
    # block maximum, which is below 8 * 2^e).
    x = np.random.default_rng(3).standard_normal((64, 512)).astype(np.float32)
    t = ref.quantize(x)
    m = ref.mxfp4_from_nvfp4(t)
    X = np.repeat(ref.e8m0_decode(m.scales), 32, axis=1) * float(t.global_scale[0])
    err = np.abs(ref.mx_dequantize(m) - ref.dequantize(t))
    assert np.all(err <= 2 * X)
    rel = np.linalg.norm(ref.mx_dequantize(m) - ref.dequantize(t)) / np.linalg.norm(ref.dequantize(t))
    assert 0.0 < rel < 0.2


def test_cols_must_be_a_multiple_of_32():
    t = _nv(np.zeros((1, 16), np.uint8), [[ONE]])
    with pytest.raises(ValueError):
        ref.mxfp4_from_nvfp4(t)
