"""GPU parity of nvfp4_gemm_nvfp4_out (GEMM whose output is quantized to NVFP4 in the same
launch, under a given output global scale).

For every output element the kernel's fp32 value is the one the same kernel stores as fp32
output (nvfp4_gemm_fused_segments with out_dtype float32, same shape, same accumulation
order); those fp32 values are checked against the oracle's Y within 1e-4 * sum_k |a_k w_k|,
then the oracle quantizes them in GIVEN mode, and codes and scale bytes must match bit for
bit.  Both prefill tile sizes (256 and the peeled 128 columns), fused
segments, and both decode kernels (K a multiple of 256, and K / 128 odd) are covered."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_gemm_close, assert_quant_equal, nv, to_gpu

pytestmark = pytest.mark.gpu


def _weights(seed, widths, K, sigma=0.02, oracle=None):
    """Quantized weight segments on the GPU; with a list for ``oracle``, the oracle's
    quantizations of the same bf16 weights are appended to it (and checked bit-exact)."""
    gq, codes, scales, globs = [], [], [], []
    for i, n in enumerate(widths):
        wg = to_gpu(workloads.weight(seed, 50 + i, n, K, sigma=sigma * (1 + 0.5 * i)))
        q = nv().quantize(wg)
        if oracle is not None:
            o = ref.quantize(wg.float().cpu().numpy())
            assert_quant_equal(q, o, what=f"w{i}")
            oracle.append(o)
        codes.append(q.codes)
        scales.append(q.scales)
        globs.append(q.global_scale)
    return torch.cat(codes), torch.cat(scales), torch.cat(globs)


def _check(M, K, widths, a_mode="per_tensor", rows=None, y_scale_factor=1.0, seed=41):
    x = workloads.activation(seed, M, M, K, outlier_frac=0.01)
    xg = to_gpu(x)
    a = nv().quantize(xg, a_mode)
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW if a_mode == "per_row" else ref.PER_TENSOR)
    assert_quant_equal(a, oa, what="x")
    ows = []
    wc, ws, wg = _weights(seed, widths, K, oracle=ows)
    y32 = nv().gemm_fused_segments(a, wc, ws, widths, wg, torch.float32)
    ysel = y32 if rows is None else y32[torch.from_numpy(rows).to(DEV)]
    # The fp32 values the encoding starts from are themselves within the GEMM tolerance.
    Y, T = ref.fused_segments(oa, ows, rows)
    assert_gemm_close(ysel, Y, T, f"fp32 values M={M} K={K} widths={widths} {a_mode}")
    yh = ysel.cpu().numpy()
    amax = float(np.max(np.abs(y32.cpu().numpy()))) if rows is None else float(y32.abs().max().item())
    s = np.float32(amax / 2688.0 * y_scale_factor)
    yq = nv().gemm_nvfp4_out(a, wc, ws, widths, wg, torch.tensor([s], dtype=torch.float32, device=DEV))
    want = ref.quantize(yh, ref.GIVEN, float(s))
    got_c, got_s = yq.codes, yq.scales
    if rows is not None:
        sel = torch.from_numpy(rows).to(DEV)
        got_c, got_s = got_c[sel], got_s[sel]
    got_c, got_s = got_c.cpu().numpy(), got_s.cpu().numpy()
    bad = np.argwhere(got_s != want.scales)
    assert bad.size == 0, f"{len(bad)} scale bytes differ, first {bad[:3].tolist()}"
    bad = np.argwhere(got_c != want.codes)
    assert bad.size == 0, f"{len(bad)} code bytes differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("M,K,widths", [(300, 512, (256,)), (257, 256, (48, 80, 128)), (40, 1024, (2064,)),
                                        (33, 768, (16,))])
def test_prefill_path(M, K, widths):
    _check(M, K, widths)


def test_prefill_per_row_activation_scale():
    _check(64, 512, (512,), a_mode="per_row")


def test_prefill_full_shape_sampled_rows():
    # 4096 x 17408 x 5120: 256 x 256 tiles plus the last columns as 128 x 128 tiles.
    p = workloads.PREFILL
    rows = np.concatenate([[0, 1, 255, 256, 4095], np.random.default_rng(7).choice(4096, 27, replace=False)])
    x = to_gpu(p.x())
    a = nv().quantize(x)
    wt = to_gpu(p.w())
    w = nv().quantize(wt)
    y32 = nv().gemm(a, w, torch.float32)
    oa, ow = ref.quantize(x.float().cpu().numpy()), ref.quantize(wt.float().cpu().numpy())
    assert_quant_equal(a, oa, what="x")
    assert_quant_equal(w, ow, what="w")
    Y, T = ref.gemm(oa, ow, rows)
    assert_gemm_close(y32[torch.from_numpy(rows).to(DEV)], Y, T, "fp32 values, prefill")
    s = np.float32(float(y32.abs().max().item()) / 2688.0)
    sg = torch.tensor([s], dtype=torch.float32, device=DEV)
    yq = nv().gemm_nvfp4_out(a, w.codes, w.scales, (p.N,), w.global_scale, sg)
    sel = torch.from_numpy(rows).to(DEV)
    want = ref.quantize(y32[sel].cpu().numpy(), ref.GIVEN, float(s))
    assert np.array_equal(yq.scales[sel].cpu().numpy(), want.scales)
    assert np.array_equal(yq.codes[sel].cpu().numpy(), want.codes)


@pytest.mark.parametrize("M,K,widths", [(1, 2048, (96,)), (7, 384, (48, 48)), (16, 4096, (1024,)),
                                        (16, 640, (32, 16)), (16, 1024, (12288,)), (3, 512, (4096, 1024, 3072))])
@pytest.mark.parametrize("a_mode", ["per_tensor", "per_row"])
def test_decode_path(M, K, widths, a_mode):
    _check(M, K, widths, a_mode=a_mode)


def test_saturating_output_scale():
    # An output scale 20x too small: most blocks saturate at E4M3 448 and E2M1 6.
    _check(64, 256, (128,), y_scale_factor=0.05)


def test_errors_and_empty():
    x = nv().quantize(to_gpu(workloads.activation(43, 0, 32, 256)))
    wc, ws, wg = _weights(43, (40,), 256)
    sg = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    with pytest.raises(nv().NVFP4Error):           # N % 16 != 0
        nv().gemm_nvfp4_out(x, wc, ws, (40,), wg, sg)
    wc2, ws2, wg2 = _weights(43, (48,), 272)
    x2 = nv().quantize(to_gpu(workloads.activation(43, 1, 32, 272)))
    with pytest.raises(nv().NVFP4Error):           # K not a multiple of 128
        nv().gemm_nvfp4_out(x2, wc2, ws2, (48,), wg2, sg)
    e = nv().quantize(torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV), "per_row")
    wc3, ws3, wg3 = _weights(43, (48,), 256)
    out = nv().gemm_nvfp4_out(e, wc3, ws3, (48,), wg3, sg)
    assert out.codes.shape == (0, 24) and out.scales.shape == (0, 3)
