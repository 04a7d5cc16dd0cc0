"""Pins for the oracle's NVFP4 encoder: hand-worked blocks, the exhaustive code x scale
round trip, idempotence, outlier locality, the global-scale rule and edge cases."""
import os

import numpy as np
import pytest

from oracle import nvfp4_ref as ref
import workloads


def _parse_golden(path):
    blocks, cur = {}, None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            cur = blocks.setdefault(line.strip("[]"), {})
            continue
        k, v = (s.strip() for s in line.split("=", 1))
        cur[k] = v
    return blocks


def test_golden_worked_blocks(golden_dir):
    blocks = _parse_golden(os.path.join(golden_dir, "worked_blocks.txt"))
    assert len(blocks) == 8
    for name, b in blocks.items():
        x = np.array([float(t) for t in b["x"].split()], dtype=np.float32)[None, :]
        mode = b["mode"].split()
        if mode[0] == "given":
            q = ref.quantize(x, ref.GIVEN, float(mode[1]))
        else:
            q = ref.quantize(x, ref.PER_TENSOR)
            assert q.global_scale[0] == np.float32(b["global"]), name
        codes = ref.unpack_codes(q.codes)[0]
        want = [int(t, 16) for t in b["codes"].split()]
        assert q.scales[0, 0] == int(b["scale"], 16), name
        assert codes.tolist() == want, name


def _exhaustive_blocks(sg: np.float32):
    """One block per nonzero finite scale byte s holding all sixteen codes c at value
    E2M1(c) * fl32(E4M3(s) * s_g).  The +-6 entries make s the block's own scale."""
    s_bytes = np.arange(1, 0x7F, dtype=np.int64)
    d = (ref.e4m3_decode(s_bytes).astype(np.float32) * sg).astype(np.float32)
    vals = ref.e2m1_decode(np.arange(16)).astype(np.float32)
    x = (vals[None, :] * d[:, None]).astype(np.float32)
    return s_bytes, x


@pytest.mark.parametrize("sg", [1.0, 2.0 ** -7, 0.37, 3.0e-5, 2.0 ** 20, 1.7e-3])
def test_every_code_with_every_scale_round_trips(sg):
    sg = np.float32(sg)
    s_bytes, x = _exhaustive_blocks(sg)
    q = ref.quantize(x.reshape(1, -1), ref.GIVEN, sg)
    assert np.array_equal(q.scales[0].astype(np.int64), s_bytes)
    codes = ref.unpack_codes(q.codes).reshape(-1, 16)
    assert np.array_equal(codes, np.tile(np.arange(16, dtype=np.uint8), (s_bytes.size, 1)))


def test_zero_scale_block_is_sign_only():
    x = np.zeros((1, 16), np.float32)
    x[0, 3] = -0.0
    x[0, 5] = -1e-45    # smallest negative denormal
    q = ref.quantize(x, ref.GIVEN, 1.0)
    assert q.scales[0, 0] == 0
    codes = ref.unpack_codes(q.codes)[0]
    assert codes[3] == 8 and codes[5] == 8 and (np.delete(codes, [3, 5]) == 0).all()


def _random_x(seed, rows=64, cols=512):
    return workloads.activation(seed, 0, rows, cols, outlier_frac=0.01, outlier_gain=50.0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_idempotent_with_fixed_global_scale(seed):
    x = _random_x(seed)
    q1 = ref.quantize(x, ref.PER_TENSOR)
    sg = q1.global_scale[0]
    x2 = ref.dequantize_f32(q1)
    q2 = ref.quantize(x2, ref.GIVEN, sg)
    keep = q1.scales >= 0x03     # block max is then exactly +-6 after dequantization
    assert keep.mean() > 0.99
    assert np.array_equal(q1.scales[keep], q2.scales[keep])
    c1 = ref.unpack_codes(q1.codes).reshape(x.shape[0], -1, 16)
    c2 = ref.unpack_codes(q2.codes).reshape(x.shape[0], -1, 16)
    assert np.array_equal(c1[keep], c2[keep])


def test_idempotent_with_rederived_global_scale():
    x = _random_x(3)
    q1 = ref.quantize(x, ref.PER_TENSOR)
    q2 = ref.quantize(ref.dequantize_f32(q1), ref.PER_TENSOR)
    assert abs(q2.global_scale[0] / q1.global_scale[0] - 1) < 1e-6
    assert (q1.scales == q2.scales).mean() > 0.999


def test_global_scale_rule():
    # amax = 2688 * 2^k gives s_g = 2^k exactly, and the block holding amax gets 448.
    for k in (-20, -3, 0, 5):
        x = np.zeros((2, 32), np.float32)
        x[1, 17] = -2688.0 * 2.0 ** k
        x[0, 2] = 3.0 * 2.0 ** k
        q = ref.quantize(x, ref.PER_TENSOR)
        assert q.global_scale[0] == np.float32(2.0 ** k)
        assert q.scales[1, 1] == 0x7E
    x = _random_x(4)
    q = ref.quantize(x, ref.PER_TENSOR)
    a = np.abs(x).reshape(x.shape[0], -1, 16).max(axis=2)
    r, j = np.unravel_index(np.argmax(a), a.shape)
    assert q.scales[r, j] == 0x7E
    # No block scale ever exceeds the largest one.
    assert q.scales.max() == 0x7E


def test_per_row_equals_per_tensor_of_each_row():
    x = _random_x(5, rows=9, cols=256)
    qr = ref.quantize(x, ref.PER_ROW)
    for r in range(x.shape[0]):
        qt = ref.quantize(x[r:r + 1], ref.PER_TENSOR)
        assert qr.global_scale[r] == qt.global_scale[0]
        assert np.array_equal(qr.codes[r], qt.codes[0])
        assert np.array_equal(qr.scales[r], qt.scales[0])


def test_outlier_is_confined_to_its_block():
    # Block scaling confines an outlier to its own block of sixteen ("The deep dive").
    x = _random_x(6, rows=4, cols=256)
    sg = np.float32(0.05)
    q0 = ref.quantize(x, ref.GIVEN, sg)
    x1 = x.copy()
    x1[2, 37] *= 80.0
    q1 = ref.quantize(x1, ref.GIVEN, sg)
    dq = q0.scales != q1.scales
    assert dq.sum() == 1 and dq[2, 37 // 16]
    c0, c1 = ref.unpack_codes(q0.codes), ref.unpack_codes(q1.codes)
    changed = np.argwhere(c0 != c1)
    assert changed.size and all(r == 2 and c // 16 == 37 // 16 for r, c in changed)


def test_dequantization_error_bound():
    # |x - x^| <= d_j where d_j = E4M3(s_j) * s_g: the E2M1 grid spacing is at most 2 and the
    # largest |x|/d_j after E4M3 rounding of the scale is below 6.4.
    x = _random_x(7, rows=32, cols=1024)
    q = ref.quantize(x, ref.PER_TENSOR)
    xh = ref.dequantize(q)
    d = ref.e4m3_decode(q.scales) * q.global_scale[0]
    err = np.abs(xh - x.astype(np.float64)).reshape(32, -1, 16)
    assert (err <= d[:, :, None] * (1 + 1e-6)).all()
    # and the error relative to the block max is at most 1/6 of it (+ the scale rounding)
    amax = np.abs(x).reshape(32, -1, 16).max(axis=2)
    assert (err.max(axis=2) <= amax * (1 / 6 + 1 / 16 + 1e-6) + 1e-30).all()


def test_nonfinite_input_flags_and_nan_scale():
    x = _random_x(8, rows=3, cols=64)
    x[1, 5] = np.nan
    q = ref.quantize(x, ref.PER_TENSOR)
    assert q.nonfinite and np.isnan(q.global_scale[0])
    qr = ref.quantize(x, ref.PER_ROW)
    assert np.isnan(qr.global_scale[1]) and np.isfinite(qr.global_scale[[0, 2]]).all()
    x[1, 5] = np.inf
    q = ref.quantize(x, ref.PER_TENSOR)
    assert q.nonfinite and not np.isfinite(q.global_scale[0])


def test_tiny_values_keep_denormal_arithmetic():
    x = (_random_x(9, rows=2, cols=64) * np.float32(1e-36)).astype(np.float32)
    q = ref.quantize(x, ref.PER_TENSOR)
    assert q.global_scale[0] > 0 and q.global_scale[0] < np.finfo(np.float32).tiny
    assert (ref.unpack_codes(q.codes) & 7).any()


def test_packing_nibble_order():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.0    # code 7, low nibble of byte 0
    x[0, 1] = -1.0   # code 0xA, high nibble of byte 0
    q = ref.quantize(x, ref.GIVEN, 1.0)
    assert q.codes[0, 0] == 0xA7
    assert q.codes.shape == (1, 8) and q.scales.shape == (1, 1)


def test_cols_must_be_block_multiple():
    with pytest.raises(ValueError):
        ref.quantize(np.zeros((2, 24), np.float32))


def test_storage_is_4p5_bits_per_element():
    # 4-bit code + an 8-bit scale shared by 16 elements; the pages' footprint figures
    # (50.13 GiB bf16 -> 17.53 GiB, "The deep dive") imply ~24.4 G parameters at 4.5 bits.
    assert ref.nvfp4_bytes(4096, 5120, 0) * 8 == 4096 * 5120 * 4.5
    gib = 2.0 ** 30
    p_total = 50.13 * gib / 2
    p_lin = (2 * p_total - 17.53 * gib) / (2 - 4.5 / 8)
    assert 24.0e9 < p_lin < 24.8e9 and 26.5e9 < p_total < 27.2e9
