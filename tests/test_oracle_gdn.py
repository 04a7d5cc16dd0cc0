"""Pins of the oracle's GDN gate epilogue (write strength = sigmoid, log-space decay =
-exp(A_log) * softplus(y + dt_bias)) against what fixes it independently of the oracle:
closed-form values, the functions' identities, Python's own libm (math.exp, math.log1p) on
moderate arguments, the closed form of the decay factor (1 + e^z)^(-e^A_log), and an
end-to-end case whose GEMM output is known exactly, so that a swapped gate segment, a lost
segment global scale, a dropped bias or a wrong head index fails."""
import math

import numpy as np
import pytest

from oracle import nvfp4_ref as ref


def test_sigmoid_closed_forms_and_symmetry():
    assert ref.sigmoid(0.0) == 0.5
    assert ref.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    assert ref.sigmoid(-math.log(3.0)) == pytest.approx(0.25, rel=1e-15)
    y = np.random.default_rng(0).standard_normal(10_000) * 20
    assert np.allclose(ref.sigmoid(y) + ref.sigmoid(-y), 1.0, rtol=0, atol=1e-15)
    # Far tails: no overflow, and the negative tail keeps full relative accuracy.
    assert ref.sigmoid(800.0) == 1.0 and ref.sigmoid(-800.0) == 0.0
    assert ref.sigmoid(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-15)


def test_softplus_closed_forms_and_identity():
    assert ref.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-16)
    assert ref.softplus(math.log(math.e - 1.0)) == pytest.approx(1.0, rel=1e-15)
    z = np.random.default_rng(1).standard_normal(10_000) * 30
    assert np.allclose(ref.softplus(z) - ref.softplus(-z), z, rtol=1e-14, atol=1e-14)
    assert ref.softplus(800.0) == 800.0
    assert ref.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-15)
    for v in (-5.0, -0.3, 0.7, 4.0, 15.0):
        assert ref.softplus(v) == pytest.approx(math.log1p(math.exp(v)), rel=1e-15)


def test_gate_values_per_head():
    # Head h gets its own A_log and dt_bias; z chosen so that softplus(z) = c_h exactly.
    c = np.array([1.0, 0.25, 3.0])
    a_log = np.array([0.0, math.log(2.0), 1.5], dtype=np.float32)
    dt = np.array([-0.5, 0.75, -2.0], dtype=np.float32)
    y_a = (np.log(np.expm1(c)) - dt.astype(np.float64))[None, :]
    y_b = np.array([[0.0, math.log(3.0), -math.log(3.0)]])
    g, beta = ref.gdn_gates(y_b, y_a, a_log, dt)
    want_g = -np.exp(a_log.astype(np.float64)) * c
    assert np.allclose(g[0], want_g, rtol=1e-14, atol=0)
    assert np.allclose(beta[0], [0.5, 0.75, 0.25], rtol=1e-15, atol=0)
    # Decay factor alpha = e^g = (1 + e^z)^(-e^A_log), an independent closed form.
    z = y_a[0] + dt
    alpha = [(1.0 + math.exp(float(zz))) ** (-math.exp(float(al))) for zz, al in zip(z, a_log)]
    assert np.allclose(np.exp(g[0]), alpha, rtol=1e-13, atol=0)


def test_gate_ranges():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((64, 48)) * 10
    a_log = rng.uniform(0.0, math.log(16.0), 48).astype(np.float32)
    dt = rng.uniform(-6.9, -2.25, 48).astype(np.float32)
    g, beta = ref.gdn_gates(y, y, a_log, dt)
    assert np.all(g < 0) and np.all(np.exp(g) <= 1.0) and np.all(np.exp(g) > 0)
    assert np.all((beta > 0) & (beta < 1))
    # g is increasing in |.| with y: a larger pre-activation decays the state more.
    g2, _ = ref.gdn_gates(y, y + 1.0, a_log, dt)
    assert np.all(g2 < g)


def _nvfp4(codes_rc: np.ndarray, scale_byte: int, global_scale: float) -> ref.NVFP4:
    R, C = codes_rc.shape
    return ref.NVFP4(ref.pack_codes(codes_rc.astype(np.uint8)),
                     np.full((R, C // 16), scale_byte, np.uint8),
                     np.asarray([global_scale], np.float32), R, C)


def test_fused_gates_end_to_end_known_gemm():
    K, H = 32, 3
    one = 0x38
    assert ref.e4m3_decode(one) == 1.0
    # A: row 0 = e_0 (code 2 = +1.0), row 1 = -e_1 (code 10 = -1.0).
    ca = np.zeros((2, K), np.uint8)
    ca[0, 0] = 2
    ca[1, 1] = 10
    a = _nvfp4(ca, one, 1.0)
    # W segments: a plain one of width 16, then b and a of width H.  Column 0 and 1 of each
    # gate row hold known E2M1 values (magnitude indices 1 = 0.5, 5 = 3, 7 = 6; bit 3 = sign).
    plain = _nvfp4(np.full((16, K), 2, np.uint8), one, 0.5)
    cb = np.zeros((H, K), np.uint8)
    cb[:, 0] = [1, 5, 8 | 7]           # 0.5, 3, -6
    cb[:, 1] = [8 | 5, 2, 0]           # -3, 1, 0
    wb = _nvfp4(cb, one, 1.0)
    cw = np.zeros((H, K), np.uint8)
    cw[:, 0] = [4, 8 | 1, 6]           # 2, -0.5, 4
    cw[:, 1] = [1, 3, 8 | 2]           # 0.5, 1.5, -1
    wa = _nvfp4(cw, one, 2.0)          # its own global scale doubles y_a
    a_log = np.array([0.0, math.log(2.0), -1.0], np.float32)
    dt = np.array([0.25, -1.0, 0.5], np.float32)
    Y, T, g, beta = ref.fused_gdn_gates(a, [plain, wb, wa], a_log, dt)

    yb = np.array([[0.5, 3.0, -6.0], [3.0, -1.0, 0.0]])          # row 1 sees -column 1
    ya = 2.0 * np.array([[2.0, -0.5, 4.0], [-0.5, -1.5, 1.0]])
    assert np.array_equal(Y[:, 16:16 + H], yb) and np.array_equal(Y[:, 16 + H:], ya)
    assert np.array_equal(Y[:, :16], np.array([[0.5] * 16, [-0.5] * 16]))
    for m in range(2):
        for h in range(H):
            assert beta[m, h] == pytest.approx(1.0 / (1.0 + math.exp(-yb[m, h])), rel=1e-15)
            sp = math.log1p(math.exp(ya[m, h] + float(dt[h])))
            assert g[m, h] == pytest.approx(-math.exp(float(a_log[h])) * sp, rel=1e-14)
    # The plain part of Y is the fused GEMM unchanged.
    Y2, T2 = ref.fused_segments(a, [plain, wb, wa])
    assert np.array_equal(Y, Y2) and np.array_equal(T, T2)


def test_fused_gates_reject_unequal_gate_widths():
    one = 0x38
    a = _nvfp4(np.zeros((1, 16), np.uint8), one, 1.0)
    w2 = _nvfp4(np.zeros((2, 16), np.uint8), one, 1.0)
    w3 = _nvfp4(np.zeros((3, 16), np.uint8), one, 1.0)
    with pytest.raises(ValueError):
        ref.fused_gdn_gates(a, [w2, w3], [0.0] * 3, [0.0] * 3)
