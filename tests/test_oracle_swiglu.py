"""Pins of the oracle's gated MLP input projection (h = silu(y_gate) * y_up, silu(y) = y *
sigmoid(y)) against what fixes it independently of the oracle: closed-form values of silu,
its minimum (which the Lambert W function gives in closed form), scipy's logistic function,
Python's libm in the tails, and an end-to-end case whose two GEMM outputs are known exactly,
so that swapped gate and up roles, a lost segment global scale or a dropped row fails."""
import math

import numpy as np
import pytest
from scipy import special

from oracle import nvfp4_ref as ref


def test_silu_closed_forms():
    ln3 = math.log(3.0)
    assert ref.silu(0.0) == 0.0
    assert ref.silu(ln3) == pytest.approx(0.75 * ln3, rel=1e-15)       # sigmoid(ln 3) = 3/4
    assert ref.silu(-ln3) == pytest.approx(-0.25 * ln3, rel=1e-15)     # sigmoid(-ln 3) = 1/4
    assert ref.silu(2.0) == pytest.approx(2.0 / (1.0 + math.exp(-2.0)), rel=1e-15)


def test_silu_minimum_is_minus_lambert_w_of_inverse_e():
    # d/dy [y sigmoid(y)] = 0 at y* = -1 - W(1/e), where the value is -W(1/e).
    w = float(special.lambertw(math.exp(-1.0)).real)
    y_star = -1.0 - w
    assert ref.silu(y_star) == pytest.approx(-w, rel=1e-14)
    grid = np.linspace(-6.0, 2.0, 200_001)
    assert ref.silu(grid).min() >= -w - 1e-15


def test_silu_tails():
    assert ref.silu(800.0) == 800.0
    assert ref.silu(-800.0) == 0.0                      # -800 e^-800 underflows; no NaN
    assert ref.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert ref.silu(-40.0) == pytest.approx(-40.0 * math.exp(-40.0), rel=1e-14)


def test_silu_against_scipy_expit():
    y = np.random.default_rng(0).standard_normal(100_000) * 15
    assert np.allclose(ref.silu(y), y * special.expit(y), rtol=1e-15, atol=0)


def _nvfp4(codes_rc: np.ndarray, scale_byte: int, global_scale: float) -> ref.NVFP4:
    R, C = codes_rc.shape
    return ref.NVFP4(ref.pack_codes(codes_rc.astype(np.uint8)),
                     np.full((R, C // 16), scale_byte, np.uint8),
                     np.asarray([global_scale], np.float32), R, C)


def test_swiglu_end_to_end_known_gemm():
    K, F = 32, 3
    one = 0x38
    assert ref.e4m3_decode(one) == 1.0
    # A: row 0 = e_0 (code 2 = +1.0), row 1 = -e_1 (code 10 = -1.0).
    ca = np.zeros((2, K), np.uint8)
    ca[0, 0] = 2
    ca[1, 1] = 10
    a = _nvfp4(ca, one, 1.0)
    # E2M1 magnitude indices: 1 = 0.5, 3 = 1.5, 4 = 2, 5 = 3, 6 = 4, 7 = 6; bit 3 = sign.
    cg = np.zeros((F, K), np.uint8)
    cg[:, 0] = [6, 8 | 4, 5]           # 4, -2, 3
    cg[:, 1] = [1, 7, 0]               # 0.5, 6, 0
    gate = _nvfp4(cg, one, 0.5)        # its own global scale halves y_gate
    cu = np.zeros((F, K), np.uint8)
    cu[:, 0] = [3, 4, 8 | 1]           # 1.5, 2, -0.5
    cu[:, 1] = [8 | 6, 2, 5]           # -4, 1, 3
    up = _nvfp4(cu, one, 2.0)          # its own global scale doubles y_up
    H, yg, tg, yu, tu = ref.swiglu_mlp(a, gate, up)

    want_g = 0.5 * np.array([[4.0, -2.0, 3.0], [-0.5, -6.0, 0.0]])     # row 1 sees -column 1
    want_u = 2.0 * np.array([[1.5, 2.0, -0.5], [4.0, -1.0, -3.0]])
    assert np.array_equal(yg, want_g) and np.array_equal(yu, want_u)
    assert np.array_equal(tg, np.abs(want_g)) and np.array_equal(tu, np.abs(want_u))
    for m in range(2):
        for j in range(F):
            g, u = want_g[m, j], want_u[m, j]
            assert H[m, j] == pytest.approx(g / (1.0 + math.exp(-g)) * u, rel=1e-15, abs=0)
    # The roles are not interchangeable: swapping gate and up changes h.
    H_swapped = ref.swiglu_mlp(a, up, gate)[0]
    assert not np.allclose(H, H_swapped)
    # Rows can be taken one at a time.
    H1 = ref.swiglu_mlp(a, gate, up, a_rows=np.array([1]))[0]
    assert np.array_equal(H1[0], H[1])


def test_swiglu_rejects_unequal_widths():
    one = 0x38
    a = _nvfp4(np.zeros((1, 16), np.uint8), one, 1.0)
    w2 = _nvfp4(np.zeros((2, 16), np.uint8), one, 1.0)
    w3 = _nvfp4(np.zeros((3, 16), np.uint8), one, 1.0)
    with pytest.raises(ValueError):
        ref.swiglu_mlp(a, w2, w3)
