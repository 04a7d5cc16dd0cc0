"""GPU parity of nvfp4_gemm_fused_gdn_gates against the oracle's fused GDN gates: Y within
1e-4 * sum_k |a_k w_k| (plus half a bf16 ulp for bf16 output) and bitwise equal to what
nvfp4_gemm_fused_segments writes; the log decay g and the write strength beta within the
bound derived in tests.gpu_helpers.gate_bounds.  Cases: the MFMA prefill kernel (gate columns
inside one tile, straddling two tiles, in the peeled 128-wide tiles of the full fused GDN
shape, H not a multiple of 16, ragged M, per-row activation scales), both decode kernels, the
plain kernel, and saturated gates."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_gates_close, assert_gemm_close, assert_quant_equal, nv, to_gpu

pytestmark = pytest.mark.gpu


def _gate_params(seed: int, H: int):
    a_log = workloads.rng(seed, 50).uniform(0.0, np.log(16.0), H).astype(np.float32)
    dt = workloads.rng(seed, 51).uniform(-6.9, -2.25, H).astype(np.float32)
    return a_log, dt


def _weights(seed, K, widths, sigmas):
    gq, oq = [], []
    for i, (n, s) in enumerate(zip(widths, sigmas)):
        wg = to_gpu(workloads.weight(seed, 1 + i, n, K, sigma=s))
        q = nv().quantize(wg)
        o = ref.quantize(wg.float().cpu().numpy())
        assert_quant_equal(q, o, what=f"w{i}")
        gq.append(q)
        oq.append(o)
    return (gq, oq, torch.cat([q.codes for q in gq]), torch.cat([q.scales for q in gq]),
            torch.cat([q.global_scale for q in gq]))


def _run(M, K, widths, seed, a_mode="per_tensor", gate_sigma=0.05, out_dtype=torch.float32, rows=None,
         x=None, params=None, sigmas=None):
    x = workloads.activation(seed, 0, M, K, outlier_frac=0.001, outlier_gain=50.0) if x is None else x
    xg = to_gpu(x)
    a = nv().quantize(xg, a_mode)
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW if a_mode == "per_row" else ref.PER_TENSOR)
    assert_quant_equal(a, oa, what="x")
    sigmas = sigmas or [0.02] * (len(widths) - 2) + [gate_sigma] * 2
    _, oq, codes, scales, globals_ = _weights(seed, K, widths, sigmas)
    H = widths[-1]
    a_log, dt = params if params is not None else _gate_params(seed, H)
    y, g, beta = nv().gemm_fused_gdn_gates(a, codes, scales, widths, globals_, torch.from_numpy(a_log).to(DEV),
                                           torch.from_numpy(dt).to(DEV), out_dtype)
    torch.cuda.synchronize()
    Y, T, g_o, beta_o = ref.fused_gdn_gates(oa, oq, a_log, dt, rows)
    sel = slice(None) if rows is None else torch.from_numpy(np.asarray(rows)).to(DEV)
    what = f"M={M} K={K} widths={widths} {a_mode} {out_dtype}"
    assert_gemm_close(y[sel], Y, T, what)
    assert_gates_close(g[sel], beta[sel], Y, T, H, a_log, dt, g_o, beta_o, what)
    # Y is the fused GEMM's output, bit for bit.
    y2 = nv().gemm_fused_segments(a, codes, scales, widths, globals_, out_dtype)
    assert torch.equal(y, y2), what
    return g, beta, g_o, beta_o


@pytest.mark.parametrize("M,K,widths", [
    (300, 512, (256, 64, 48, 48)),        # gates inside one 256-wide tile column
    (100, 256, (200, 48, 48)),            # gates straddle the 256-column tile boundary
    (200, 768, (512, 40, 40)),            # H not a multiple of 16, ragged last tile
    (64, 256, (96, 16, 16)),
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_prefill_gates(M, K, widths, out_dtype):
    _run(M, K, widths, seed=40 + M, out_dtype=out_dtype)


def test_prefill_gates_per_row_scales():
    _run(257, 512, (128, 48, 48), seed=47, a_mode="per_row")


@pytest.mark.parametrize("M", [1, 7, 16])
@pytest.mark.parametrize("K", [512, 384])     # 512: the LDS-streaming decode kernel; 384: the register one
def test_decode_gates(M, K):
    _run(M, K, (64, 48, 48), seed=60 + M, a_mode="per_row")


@pytest.mark.parametrize("M", [1, 16])
def test_decode_gates_full_fused_gdn_width(M):
    # The fused GDN projection's width (12384 columns) at decode: 49 rows per workgroup, four
    # row groups, the gate columns spread over the last workgroups.
    f = workloads.FUSED
    _run(M, 1024, f.widths, seed=80 + M, a_mode="per_row")


def test_plain_kernel_gates():
    # K not a multiple of 128: the plain kernel.
    _run(20, 144, (32, 24, 24), seed=70)


def test_saturated_gates():
    # Gate weights ten times larger: pre-activations of tens to hundreds, beta at 0 or 1,
    # softplus deep in both tails.
    g, beta, g_o, beta_o = _run(128, 512, (64, 48, 48), seed=71, gate_sigma=0.5)
    b = beta.cpu().numpy()
    assert (b == 0.0).any() and (b == 1.0).any() and np.isfinite(g.cpu().numpy()).all()


def test_full_fused_gdn_shape_sampled_rows():
    f = workloads.FUSED
    rows = np.concatenate([[0, f.M - 1], np.random.default_rng(8).choice(f.M, 40, replace=False)])
    _run(f.M, f.K, f.widths, seed=f.seed, out_dtype=torch.bfloat16, rows=rows, x=f.x(),
         params=f.gate_params(), sigmas=list(f.sigmas))
