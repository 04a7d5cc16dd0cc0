"""GPU parity of the GEMM over seeded random shapes that reach every kernel the launcher can
pick: the batch-1 matrix-vector kernel (M = 1, K % 64 == 0), the plain kernel (K % 128 != 0,
or more than 16 tokens with K % 256 != 0), the register decode kernel (M <= 16, K % 256 != 0),
the K-split and balanced decode kernels (M <= 16, K % 256 == 0, N on either side of one round of
32-row workgroups) and the prefill tiles with their peeled 128 x 128 tails.  Each case is a
fused launch of 1-4 modules with their own global scales (one module: the plain GEMM), per-
tensor or per-row activation scales and fp32 or bf16 output, checked element by element against
the oracle's fused GEMM with the per-element bound of the other parity tests."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import assert_gemm_close, assert_quant_equal, nv, to_gpu

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(2024)
    cases = []
    # (M range, N range, K choices) per dispatch class
    classes = [
        ("batch-1", (1, 1), (1, 700), [64, 192, 320, 576, 2112, 4160]),
        ("plain K", (1, 40), (1, 200), [16, 48, 80, 144, 208, 400]),
        ("plain M>16", (17, 70), (1, 200), [128, 384, 640]),
        ("register decode", (2, 16), (1, 300), [128, 384, 896]),
        ("K-split decode", (2, 16), (1, 900), [256, 512, 1280, 2304]),
        ("balanced decode", (1, 16), (8193, 9400), [256, 512]),
        ("prefill tiles", (17, 300), (1, 700), [256, 512, 768]),
    ]
    for name, (m0, m1), (n0, n1), ks in classes:
        for _ in range(10):
            M = int(rng.integers(m0, m1 + 1))
            N = int(rng.integers(n0, n1 + 1))
            K = int(rng.choice(ks))
            nseg = int(rng.integers(1, 5)) if N >= 4 else 1
            cuts = sorted(rng.choice(np.arange(1, N), size=nseg - 1, replace=False).tolist()) if nseg > 1 else []
            widths = [b - a for a, b in zip([0] + cuts, cuts + [N])]
            mode = "per_row" if rng.random() < 0.5 else "per_tensor"
            out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
            seed = int(rng.integers(0, 1 << 30))
            cases.append(pytest.param(M, K, tuple(widths), mode, out, seed, id=f"{name}-{M}x{N}x{K}-{len(widths)}seg"))
    return cases


@pytest.mark.parametrize("M,K,widths,mode,out_dtype,seed", _cases())
def test_random_shape(M, K, widths, mode, out_dtype, seed):
    xg = to_gpu(workloads.activation(seed, 0, M, K))
    a = nv().quantize(xg, mode)
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW if mode == "per_row" else ref.PER_TENSOR)
    assert_quant_equal(a, oa, what="A")
    gq, oq = [], []
    for i, n in enumerate(widths):
        wg = to_gpu(workloads.weight(seed, 1 + i, n, K, sigma=0.02 * (1 + i)))
        gq.append(nv().quantize(wg))
        oq.append(ref.quantize(wg.float().cpu().numpy()))
        assert_quant_equal(gq[-1], oq[-1], what=f"W{i}")
    if len(widths) == 1:
        y = nv().gemm(a, gq[0], out_dtype)
    else:
        y = nv().gemm_fused_segments(a, torch.cat([q.codes for q in gq]), torch.cat([q.scales for q in gq]),
                                     widths, torch.cat([q.global_scale for q in gq]), out_dtype)
    Y, T = ref.fused_segments(oa, oq)
    assert_gemm_close(y, Y, T, f"M={M} K={K} widths={widths} {mode}")
