"""GPU parity of every GEMM kernel over every E4M3 block-scale byte, 0x00 to 0x7E.

The block scale is an E4M3 byte per 16 elements ("NVFP4 W4A4 Quantization Compresses 27B
Hybrid Models", "Challenging the Recurrence Fragility Assumption"); the quantizer can emit any
byte except the NaN 0x7F, including the subnormal bytes 0x01 to 0x07 (2^-9 to 7 * 2^-9) and
zero.  Each operand row here carries one byte for all of its blocks, and the rows cycle
through all 127 bytes, so every output element is the product of exactly one A byte and one
W byte: a byte that a kernel decoded wrongly (a subnormal flushed to zero, say) changes whole
output rows or columns by far more than the tolerance 1e-4 * sum_k |a_k w_k| (plus half a bf16
ulp for bf16 output).  Every pair of bytes meets in every kernel family: the prefill kernel's
256 x 256 tiles and its peeled 128 x 128 tiles, the K-split decode kernel on 16 x 16 x 32 MFMAs
and on 4 x 4 x 4 MFMAs (up to 4 tokens, four or five 4-row groups), the balanced (three to five
row groups, and the SwiGLU pairs) and register decode kernels, the plain kernel; fp32 and bf16
output, and the NVFP4-output, GDN gate and SwiGLU epilogues.

Codes are seeded random bytes and the same bytes go to the GPU and the oracle.  With K = 256
every partial sum is an integer multiple of 2^(e-8) below 2^24 units, so the kernel's fp32
accumulator is exact and the comparison tests the decoding of the bytes, not rounding."""
import numpy as np
import pytest
import torch

from oracle import nvfp4_ref as ref
from tests.gpu_helpers import (DEV, assert_gates_close, assert_gemm_close, assert_swiglu_close, nv,
                               to_device)

pytestmark = pytest.mark.gpu

NBYTES = 0x7F          # bytes 0x00 .. 0x7E: every non-negative E4M3FN byte that is not NaN


def _operand(seed, R, K, offset, gs):
    """R rows of random codes; row r has scale byte (r + offset) mod 127 in every block."""
    g = np.random.default_rng(seed)
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    byte = ((np.arange(R) + offset) % NBYTES).astype(np.uint8)
    scales = np.ascontiguousarray(np.repeat(byte[:, None], K // 16, axis=1))
    return ref.NVFP4(codes, scales, np.asarray(gs, np.float32).reshape(-1), R, K)


def _a_operand(seed, M, K, offset, per_row):
    gs = np.random.default_rng(seed + 1).uniform(0.5, 2.0, M if per_row else 1)
    return _operand(seed, M, K, offset, gs)


def _check_store(oa, ow, what):
    a, w = to_device(oa), to_device(ow)
    Y, T = ref.gemm(oa, ow)
    for dt in (torch.float32, torch.bfloat16):
        y = nv().gemm(a, w, dt)
        assert_gemm_close(y, Y, T, f"{what} {dt}")


def _assert_all_pairs(oa_list, ow):
    """Every (A byte, W byte) pair occurs among the operands."""
    a_bytes = np.unique(np.concatenate([o.scales[:, 0] for o in oa_list]))
    assert a_bytes.size == NBYTES and np.unique(ow.scales[:, 0]).size == NBYTES


@pytest.mark.parametrize("per_row", [False, True])
def test_prefill_tiles_every_byte(per_row):
    # M = 200, N = 257 * 256: one tile row of 257 tiles on 256 CUs, so the last 256 columns
    # are peeled into 128 x 128 tiles (two tile rows, the second ragged).
    M, N, K = 200, 257 * 256, 256
    oa = _a_operand(11, M, K, 0, per_row)
    ow = _operand(12, N, K, 5, [0.75])
    _assert_all_pairs([oa], ow)
    _check_store(oa, ow, f"prefill per_row={per_row}")


def _decode_launches(seed, N, K, per_row=True):
    """Eight 16-token activations whose rows cover all 127 bytes, and one weight."""
    ow = _operand(seed, N, K, 3, [1.25])
    oas = [_a_operand(seed + 10 + j, 16, K, 16 * j, per_row) for j in range(8)]
    _assert_all_pairs(oas, ow)
    return oas, ow


# N <= 32 * CUs with K % 256 == 0: the K-split kernel; N = 12000 / 16000 / 20000: the balanced
# kernel with 47 / 63 / 79 rows per workgroup (three, four and five 16-row groups on 256 CUs);
# K = 384 (K / 128 odd): the register kernel.
@pytest.mark.parametrize("N,K", [(1000, 512), (12000, 256), (16000, 256), (20000, 256), (1000, 384)])
def test_decode_kernels_every_byte(N, K):
    oas, ow = _decode_launches(20 + N + K, N, K)
    for j, oa in enumerate(oas):
        _check_store(oa, ow, f"decode N={N} K={K} launch {j}")


# Up to 4 tokens with at most 20 rows per workgroup (N <= 20 x CUs): the K-split kernel on
# 4 x 4 x 4 MFMAs, with four row groups (N = 1000: 16 rows per workgroup on 256 CUs) and five
# (N = 4700: 19 rows, so the last group holds three real rows).  3 and 4 tokens per launch.
# 5 to 8 tokens: the 16 x 16 x 32 K-split kernel copying one token chunk, with three W chunks
# (N = 6000: 24 rows per workgroup on 256 CUs) and four (N = 8000: 32 rows).
@pytest.mark.parametrize("N,M", [(1000, 4), (4700, 3), (6000, 8), (8000, 6)])
def test_small_batch_decode_every_byte(N, M):
    K = 256
    ow = _operand(70 + N, N, K, 3, [1.25])
    oas = [_a_operand(71 + N + j, M, K, M * j, True) for j in range((NBYTES + M - 1) // M)]
    _assert_all_pairs(oas, ow)
    for j, oa in enumerate(oas):
        _check_store(oa, ow, f"small-batch decode N={N} M={M} launch {j}")


@pytest.mark.parametrize("M", [16, 127])
def test_plain_kernel_every_byte(M):
    # K % 128 != 0: the plain kernel, for decode-sized and larger M.
    K = 112
    ow = _operand(31, 300, K, 0, [0.5])
    oas = [_a_operand(32 + j, M, K, M * j, True) for j in range((NBYTES + M - 1) // M)]
    _assert_all_pairs(oas, ow)
    for j, oa in enumerate(oas):
        _check_store(oa, ow, f"plain M={M} launch {j}")


def _check_nvfp4_out(oa, ow, what):
    """The NVFP4-output epilogue: the same launch's fp32 values within tolerance of the oracle,
    and the NVFP4 output equal to the oracle's GIVEN-mode encoding of those values."""
    a, w = to_device(oa), to_device(ow)
    Y, T = ref.gemm(oa, ow)
    y32 = nv().gemm(a, w, torch.float32)
    assert_gemm_close(y32, Y, T, f"{what} fp32")
    s = np.float32(float(y32.abs().max().item()) / 2688.0)
    yq = nv().gemm_nvfp4_out(a, w.codes, w.scales, (ow.rows,), w.global_scale,
                             torch.tensor([s], dtype=torch.float32, device=DEV))
    want = ref.quantize(y32.cpu().numpy(), ref.GIVEN, float(s))
    assert np.array_equal(yq.scales.cpu().numpy(), want.scales), what
    assert np.array_equal(yq.codes.cpu().numpy(), want.codes), what


def test_nvfp4_out_prefill_every_byte():
    oa = _a_operand(41, 200, 256, 0, True)
    ow = _operand(42, 257 * 256, 256, 9, [0.75])
    _check_nvfp4_out(oa, ow, "nvfp4 out prefill")


@pytest.mark.parametrize("N", [1024, 12288])
def test_nvfp4_out_decode_every_byte(N):
    oas, ow = _decode_launches(43 + N, N, 256)
    for j, oa in enumerate(oas):
        _check_nvfp4_out(oa, ow, f"nvfp4 out decode N={N} launch {j}")


def _check_gates(oa, ows, what):
    widths = tuple(o.rows for o in ows)
    H = widths[-1]
    a_log = np.random.default_rng(7).uniform(0.0, np.log(16.0), H).astype(np.float32)
    dt = np.random.default_rng(8).uniform(-6.9, -2.25, H).astype(np.float32)
    a = to_device(oa)
    wc = torch.cat([to_device(o).codes for o in ows])
    ws = torch.cat([to_device(o).scales for o in ows])
    wg = torch.from_numpy(np.concatenate([o.global_scale for o in ows]).astype(np.float32)).to(DEV)
    y, g, beta = nv().gemm_fused_gdn_gates(a, wc, ws, widths, wg, torch.from_numpy(a_log).to(DEV),
                                           torch.from_numpy(dt).to(DEV), torch.float32)
    Y, T, g_o, beta_o = ref.fused_gdn_gates(oa, ows, a_log, dt)
    assert_gemm_close(y, Y, T, what)
    assert_gates_close(g, beta, Y, T, H, a_log, dt, g_o, beta_o, what)


@pytest.mark.parametrize("M", [200, 16, 4])
def test_gates_every_byte(M):
    # Three segments: 381 plain columns, then the two 127-wide gate projections; each gate
    # column has its own byte, so every byte reaches both gate functions.
    K = 256
    ows = [_operand(51, 381, K, 0, [0.02]), _operand(52, 127, K, 0, [0.01]), _operand(53, 127, K, 40, [0.01])]
    oas = [_a_operand(54 + j, M, K, M * j, True) for j in range((NBYTES + M - 1) // M)]
    for j, oa in enumerate(oas):
        _check_gates(oa, ows, f"gates M={M} launch {j}")


def _check_swiglu(oa, og, ou, what):
    a, gate, up = to_device(oa), to_device(og), to_device(ou)
    wc, ws = nv().interleave_gate_up(gate, up)
    wg = torch.cat([gate.global_scale, up.global_scale])
    H, yg, tg, yu, tu = ref.swiglu_mlp(oa, og, ou)
    h, _ = nv().gemm_swiglu(a, wc, ws, wg, h_dtype=torch.float32)
    assert_swiglu_close(h, H, yg, tg, yu, tu, what)
    hb, _ = nv().gemm_swiglu(a, wc, ws, wg, h_dtype=torch.bfloat16)
    assert_swiglu_close(hb, H, yg, tg, yu, tu, what + " bf16")


# F = 16 * 257 with M = 200 takes the prefill kernel (with peeled tiles); with M = 16 the
# balanced decode kernel's pair groups (F = 4112 > 32 * CUs / 2 rows).
@pytest.mark.parametrize("M,F", [(200, 16 * 257 * 8), (16, 4112 * 2)])
def test_swiglu_every_byte(M, F):
    K = 256
    og = _operand(61, F, K, 0, [0.02])
    ou = _operand(62, F, K, 60, [0.03])
    oas = [_a_operand(63 + j, M, K, M * j, True) for j in range((NBYTES + M - 1) // M)]
    for j, oa in enumerate(oas):
        _check_swiglu(oa, og, ou, f"swiglu M={M} F={F} launch {j}")
