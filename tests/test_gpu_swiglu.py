"""GPU parity of the gated MLP input projection (nvfp4_interleave_gate_up + nvfp4_gemm_swiglu):
the fused gate+up GEMM with its SwiGLU activation h = silu(y_gate) * y_up in the same launch.

Inputs are built on the host (seeded workload tensors quantized by the oracle, or seeded
random NVFP4 bytes for the full-size shapes) and the same bytes go to the GPU and the oracle.
h (fp32 or bf16) must lie within the bound derived from the GEMM tolerance 1e-4 * T of each
product and the slope of silu (at most 1.1 in magnitude), plus (|y_gate| + 4) 2^-23 of h for
the fp32 evaluation (hardware exponential and reciprocal, each within one ulp, on an argument
rounded to fp32), plus half a bf16 ulp for bf16.
The NVFP4 encoding of h is compared bit for bit with the oracle's GIVEN-mode quantization of
the fp32 h the same launch stores (the encoding decision is taken in the kernel's precision).
Covered: both prefill tile sizes (256 and the peeled 128 columns), ragged M and F, per-row
activation scales, all three decode kernels (K-split, K / 128 odd, balanced rows), strided and
unaligned h rows, NVFP4-only output, and gate outputs far past +-88 (the exponential overflowing
to infinity, or vanishing)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_swiglu_close, nv, to_device

pytestmark = pytest.mark.gpu


def _workload_operands(seed, M, F, K, a_mode=ref.PER_TENSOR):
    """Seeded activations (1 % hot channels) and gate/up weights, quantized by the oracle."""
    x = workloads.activation(seed, 0, M, K, outlier_frac=0.01)
    gate = workloads.weight(seed, 1, F, K)
    up = workloads.weight(seed, 2, F, K, sigma=0.03)
    return ref.quantize(x, a_mode), ref.quantize(gate), ref.quantize(up)


def _random_operands(seed, M, F, K):
    """Seeded NVFP4 bytes (random codes, block scales over 2^-5 .. 2^1, a global scale per
    token row); the weight global scales are set so that the gate outputs are of order one
    to ten, where silu bends."""
    g = np.random.default_rng(seed)

    def operand(R, gs):
        codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
        scales = g.integers(0x10, 0x40, (R, K // 16), dtype=np.uint8)
        return ref.NVFP4(codes, scales, np.asarray(gs, np.float32), R, K)

    oa = operand(M, g.uniform(0.5, 2.0, M))
    # |E2M1| has rms ~2.9 and the block scales rms ~0.6 over these bytes: one product has rms
    # ~3, a K-long sum ~3 sqrt(K) before the global scales.
    unit = 1.0 / (3.0 * np.sqrt(K))
    return oa, operand(F, [4.0 * unit]), operand(F, [2.0 * unit])


def _assert_h_close(h, H, yg, tg, yu, tu, what):
    assert_swiglu_close(h, H, yg, tg, yu, tu, what)


def _launch(oa, og, ou):
    a, gate, up = to_device(oa), to_device(og), to_device(ou)
    wc, ws = nv().interleave_gate_up(gate, up)
    wg = torch.cat([gate.global_scale, up.global_scale])
    return a, wc, ws, wg


def _check(oa, og, ou, h_dtype, rows=None, quant=True, what=""):
    """One launch with h in h_dtype (and NVFP4 h when quant); compare against the oracle on
    all rows or the given ones."""
    a, wc, ws, wg = _launch(oa, og, ou)
    H, yg, tg, yu, tu = ref.swiglu_mlp(oa, og, ou, a_rows=rows)
    s = np.float32(np.max(np.abs(H)) / 2688.0)
    hg = torch.tensor([s], dtype=torch.float32, device=DEV) if quant else None
    h, q = nv().gemm_swiglu(a, wc, ws, wg, h_dtype=h_dtype, h_global=hg)
    sel = None if rows is None else torch.from_numpy(np.asarray(rows)).to(DEV)
    hs = h if sel is None else h[sel]
    _assert_h_close(hs, H, yg, tg, yu, tu, what)
    if quant:
        qc, qs = (q.codes, q.scales) if sel is None else (q.codes[sel], q.scales[sel])
        if h_dtype == torch.float32:
            want = ref.quantize(hs.cpu().numpy(), ref.GIVEN, float(s))
        else:
            # The encoding comes from the fp32 h, which a float32 launch stores.
            h32, _ = nv().gemm_swiglu(a, wc, ws, wg, h_dtype=torch.float32)
            want = ref.quantize((h32 if sel is None else h32[sel]).cpu().numpy(), ref.GIVEN, float(s))
        bad = np.argwhere(qs.cpu().numpy() != want.scales)
        assert bad.size == 0, f"{what}: {len(bad)} scale bytes differ, first {bad[:3].tolist()}"
        bad = np.argwhere(qc.cpu().numpy() != want.codes)
        assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first {bad[:3].tolist()}"


def test_interleave_layout():
    F, K = 80, 512
    og, ou = _random_operands(3, 1, F, K)[1:]
    gate, up = to_device(og), to_device(ou)
    wc, ws = nv().interleave_gate_up(gate, up)
    wc, ws = wc.cpu().numpy(), ws.cpu().numpy()
    for p in range(F // 16):
        assert np.array_equal(wc[32 * p:32 * p + 16], og.codes[16 * p:16 * p + 16])
        assert np.array_equal(wc[32 * p + 16:32 * p + 32], ou.codes[16 * p:16 * p + 16])
        assert np.array_equal(ws[32 * p:32 * p + 16], og.scales[16 * p:16 * p + 16])
        assert np.array_equal(ws[32 * p + 16:32 * p + 32], ou.scales[16 * p:16 * p + 16])


@pytest.mark.parametrize("M,F,K,a_mode,h_dtype", [
    (300, 256, 512, ref.PER_TENSOR, torch.float32),
    (257, 208, 256, ref.PER_ROW, torch.bfloat16),     # last tile column ragged (N = 416)
    (40, 1040, 1024, ref.PER_TENSOR, torch.float32),
    (33, 16, 768, ref.PER_TENSOR, torch.bfloat16),    # one pair
])
def test_prefill(M, F, K, a_mode, h_dtype):
    oa, og, ou = _workload_operands(70 + M, M, F, K, a_mode)
    _check(oa, og, ou, h_dtype, what=f"prefill {M}x{F}x{K}")


def test_prefill_peeled_small_tiles():
    # 700 x 22016 x 256 on 256 CUs: 3 x 86 large tiles leave 2 for a last round, so the last
    # 256 columns run as 128 x 128 tiles.
    M, F, K = 700, 11008, 256
    oa, og, ou = _workload_operands(77, M, F, K)
    rows = np.array([0, 1, 127, 128, 255, 256, 511, 512, 640, 699])
    _check(oa, og, ou, torch.float32, rows=rows, what="peeled tiles")


def test_prefill_full_mlp_shape_sampled_rows():
    # The 27B model's MLP input projection at a 4096-token prefill: gate and up 17408 x 5120.
    M, F, K = 4096, 17408, 5120
    oa, og, ou = _random_operands(78, M, F, K)
    rows = np.concatenate([[0, 255, 256, 4095], np.random.default_rng(8).choice(4096, 12, replace=False)])
    _check(oa, og, ou, torch.bfloat16, rows=rows, what="full MLP prefill")


@pytest.mark.parametrize("M,F,K", [
    (1, 1024, 512), (16, 2048, 1024), (5, 48, 256),        # K-split kernel
    (3, 512, 384), (16, 96, 640),                          # K / 128 odd
    (1, 4112, 256), (9, 8448, 1024), (4, 6000, 512),       # balanced rows (2F > 32 x CUs)
])
def test_decode(M, F, K):
    oa, og, ou = _random_operands(90 + M, M, F, K)
    _check(oa, og, ou, torch.float32, what=f"decode {M}x{F}x{K}")


@pytest.mark.parametrize("M", [1, 16])
def test_decode_full_mlp_shape(M):
    oa, og, ou = _random_operands(95 + M, M, 17408, 5120)
    _check(oa, og, ou, torch.bfloat16, what=f"decode MLP M={M}")


@pytest.mark.parametrize("M,F,K", [(64, 272, 512), (7, 272, 512), (2, 4608, 256)])
@pytest.mark.parametrize("h_dtype", [torch.bfloat16, torch.float32])
def test_strided_unaligned_h(M, F, K, h_dtype):
    # Row pitch F + 1: rows are not 16-byte aligned, so h leaves through element stores.
    oa, og, ou = _random_operands(60 + M, M, F, K)
    a, wc, ws, wg = _launch(oa, og, ou)
    H, yg, tg, yu, tu = ref.swiglu_mlp(oa, og, ou)
    buf = torch.full((M, F + 1), 12345.0, dtype=h_dtype, device=DEV)
    h, _ = nv().gemm_swiglu(a, wc, ws, wg, h_dtype=h_dtype, out=buf[:, :F])
    _assert_h_close(h, H, yg, tg, yu, tu, f"strided {M}x{F}x{K}")
    assert torch.all(buf[:, F] == 12345.0), "the padding column was written"


@pytest.mark.parametrize("M,F,K", [(48, 512, 512), (6, 512, 512), (3, 5008, 256)])
def test_nvfp4_only_output(M, F, K):
    oa, og, ou = _random_operands(50 + M, M, F, K)
    a, wc, ws, wg = _launch(oa, og, ou)
    hg = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    h32, q_both = nv().gemm_swiglu(a, wc, ws, wg, h_dtype=torch.float32, h_global=hg)
    none, q_only = nv().gemm_swiglu(a, wc, ws, wg, h_dtype=None, h_global=hg)
    assert none is None
    assert torch.equal(q_only.codes, q_both.codes) and torch.equal(q_only.scales, q_both.scales)
    want = ref.quantize(h32.cpu().numpy(), ref.GIVEN, 0.01)
    assert np.array_equal(q_only.scales.cpu().numpy(), want.scales)
    assert np.array_equal(q_only.codes.cpu().numpy(), want.codes)


@pytest.mark.parametrize("M,F,K", [(300, 512, 512), (5, 512, 512), (3, 4608, 512)])
def test_extreme_gate_values(M, F, K):
    # Gate outputs spread over several hundred: e^-y overflows to infinity for y < -88 (silu flushes
    # to -0) and vanishes for y > 88 (silu(y) = y); prefill, K-split and balanced decode kernels.
    oa, og, ou = _random_operands(40 + M, M, F, K)
    og = ref.NVFP4(og.codes, og.scales, og.global_scale * np.float32(40.0), og.rows, og.cols)
    H, yg, _, _, _ = ref.swiglu_mlp(oa, og, ou)
    assert (yg < -88).mean() > 0.1 and (yg > 88).mean() > 0.1
    _check(oa, og, ou, torch.float32, what=f"extreme gates {M}x{F}x{K}")


def test_rejects_shapes_without_mfma_kernel():
    oa, og, ou = _random_operands(1, 32, 64, 384)
    a, wc, ws, wg = _launch(oa, og, ou)
    with pytest.raises(nv().NVFP4Error):
        nv().gemm_swiglu(a, wc, ws, wg)          # M > 16 needs K % 256 == 0
