"""Pins for the oracle's block-scaled GEMM and fused-segment GEMM: exact rational dot
products on the tiny workload, an integer special case against int64 matmul, the fused ==
separate identity and the exact factor of the global-scale mismatch."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_ref as ref
import workloads


def _frac_e2m1(c):
    s, e, m = c >> 3, (c >> 1) & 3, c & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * Fraction(2 + m, 2)
    return -mag if s else mag


def _frac_e4m3(b):
    e, m = (b >> 3) & 15, b & 7
    return Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def _exact_dequant(t: ref.NVFP4):
    """Rational dequantization written from the bit definitions (no oracle tables)."""
    rows = []
    g = t.global_per_row()
    for r in range(t.rows):
        row = []
        for i in range(t.cols):
            byte = int(t.codes[r, i // 2])
            c = byte & 0xF if i % 2 == 0 else byte >> 4
            row.append(_frac_e2m1(c) * _frac_e4m3(int(t.scales[r, i // 16])) * Fraction(float(g[r])))
        rows.append(row)
    return rows


def test_tiny_gemm_matches_exact_rationals():
    cfg = workloads.TINY
    a = ref.quantize(cfg.x(), ref.PER_TENSOR)
    w = ref.quantize(cfg.w(), ref.PER_TENSOR)
    Y, T = ref.gemm(a, w)
    A, W = _exact_dequant(a), _exact_dequant(w)
    cols = range(0, cfg.N, 4)        # every 4th output column keeps this a few seconds
    worst = 0.0
    for m in range(cfg.M):
        for n in cols:
            exact = sum(x * y for x, y in zip(A[m], W[n]))
            tol = sum(abs(x * y) for x, y in zip(A[m], W[n]))
            # float64 sums of K terms: error at most K * 2^-53 of the absolute sum
            assert abs(float(tol) - T[m, n]) <= cfg.K * 2.0 ** -53 * float(tol)
            worst = max(worst, abs(float(Fraction(Y[m, n]) - exact)) / float(tol))
    assert worst <= cfg.K * 2.0 ** -53


def test_tiny_quantization_error_is_plausible():
    # Context only (parity unpinned for synthetic data): NVFP4 W4A4 relative GEMM error on
    # the tiny workload is a few percent of |Y|, in the range the pages report for real
    # projections (about 8-11 % on the gate GEMMs, "The deep dive").
    cfg = workloads.TINY
    x, w = cfg.x(), cfg.w()
    Y, _ = ref.gemm(ref.quantize(x), ref.quantize(w))
    Y0 = x.astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(Y - Y0) / np.linalg.norm(Y0)
    assert 0.01 < rel < 0.25


def _unit_scale_tensor(codes: np.ndarray) -> ref.NVFP4:
    R, C = codes.shape
    return ref.NVFP4(ref.pack_codes(codes), np.full((R, C // 16), 0x38, np.uint8),
                     np.asarray([1.0], np.float32), R, C)


@pytest.mark.parametrize("M,N,K", [(8, 24, 64), (33, 17, 1024), (5, 64, 4096)])
def test_integer_special_case_vs_int64_matmul(M, N, K):
    # Scale bytes 0x38 (= 1.0) and global scale 1.0: every value is k/2 with k an integer in
    # [-12, 12], so Y = (2A)(2W)^T / 4 exactly.
    g = np.random.default_rng(M * N + K)
    ca = g.integers(0, 16, (M, K), dtype=np.uint8)
    cw = g.integers(0, 16, (N, K), dtype=np.uint8)
    Y, _ = ref.gemm(_unit_scale_tensor(ca), _unit_scale_tensor(cw))
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)
    ia = np.where(ca & 8, -1, 1) * twice[ca & 7]
    iw = np.where(cw & 8, -1, 1) * twice[cw & 7]
    assert np.array_equal(Y * 4, (ia @ iw.T).astype(np.float64))


def _fused_case(rows=24, K=256, widths=(64, 32, 48, 16), sigmas=(0.02, 0.015, 0.05, 0.1)):
    x = workloads.activation(11, 0, rows, K, outlier_frac=0.02)
    a = ref.quantize(x, ref.PER_TENSOR)
    segs = [ref.quantize(workloads.weight(11, 1 + i, n, K, sigma=s), ref.PER_TENSOR)
            for i, (n, s) in enumerate(zip(widths, sigmas))]
    return a, segs


def test_fused_equals_separate():
    a, segs = _fused_case()
    Yf, Tf = ref.fused_segments(a, segs)
    off = 0
    for w in segs:
        Y, T = ref.gemm(a, w)
        assert np.array_equal(Yf[:, off:off + w.rows], Y)
        assert np.array_equal(Tf[:, off:off + w.rows], T)
        off += w.rows


def test_shared_global_scale_mismatch_factor():
    # Serving segment i with segment 0's global scale scales its outputs by s_g0 / s_gi.
    a, segs = _fused_case()
    Yg, Tg = ref.fused_segments(a, segs)
    s0 = float(segs[0].global_scale[0])
    Yb, _ = ref.fused_shared_scale(a, segs, s0)
    off = 0
    for w in segs:
        sl = slice(off, off + w.rows)
        ratio = s0 / float(w.global_scale[0])
        # equal up to float64 rounding of the two K-term sums
        assert (np.abs(Yb[:, sl] - ratio * Yg[:, sl]) <= 1e-13 * ratio * Tg[:, sl]).all()
        off += w.rows
    # The high-variance gate-like segments come out about 2.5-5x too small.
    assert s0 / float(segs[2].global_scale[0]) < 0.5


def test_gemm_row_subset_matches_full():
    a, segs = _fused_case()
    Y, T = ref.gemm(a, segs[0])
    rows = np.array([3, 0, 17, 23])
    Ys, Ts = ref.gemm(a, segs[0], rows)
    # the BLAS may block the two products differently: equal up to float64 rounding
    assert (np.abs(Ys - Y[rows]) <= 1e-13 * T[rows]).all()
    assert (np.abs(Ts - T[rows]) <= 1e-13 * T[rows]).all()


def test_per_row_activation_scale_in_gemm():
    x = workloads.activation(12, 0, 6, 128)
    w = ref.quantize(workloads.weight(12, 1, 8, 128))
    ar = ref.quantize(x, ref.PER_ROW)
    Y, T = ref.gemm(ar, w)
    for r in range(6):
        Yr, _ = ref.gemm(ref.quantize(x[r:r + 1], ref.PER_TENSOR), w)
        assert (np.abs(Y[r] - Yr[0]) <= 1e-13 * T[r]).all()
