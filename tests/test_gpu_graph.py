"""The library under HIP graph capture: every entry point is stream-ordered, allocates nothing
and never synchronises, so a captured step must replay to exactly the eager result.  Each
graph is replayed several times with new inputs written eagerly between the replays, and every
replay is compared bitwise with an eager run on the same inputs."""
import pytest
import torch

import workloads
from tests.gpu_helpers import DEV, nv, to_gpu

pytestmark = pytest.mark.gpu


def _fill(t: torch.Tensor, seed: int, rows: int, cols: int) -> None:
    t.copy_(to_gpu(workloads.activation(seed, 0, rows, cols, outlier_frac=0.01, outlier_gain=50.0)))


def _replay_and_compare(g: torch.cuda.CUDAGraph, x: torch.Tensor, rows: int, cols: int, outputs, eager) -> None:
    for i in range(4):
        _fill(x, 300 + i, rows, cols)           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        for got, ref in zip(outputs, want):
            assert torch.equal(got, ref), f"replay {i}"


def test_graph_quantize_then_gemm():
    M, N, K = 512, 1024, 1024
    w = nv().quantize(to_gpu(workloads.weight(200, 1, N, K)))
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    _fill(x, 299, M, K)
    a = nv().quantize(x)                          # eager first: per-device set-up happens here
    y = nv().gemm(a, w, torch.bfloat16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv().quantize(x, out=a)
        nv().gemm(a, w, torch.bfloat16, out=y)

    def eager():
        ae = nv().quantize(x)
        return ae.codes, ae.scales, ae.global_scale, nv().gemm(ae, w, torch.bfloat16)

    _replay_and_compare(g, x, M, K, (a.codes, a.scales, a.global_scale, y), eager)


def test_graph_decode_per_row():
    M, N, K = 4, 512, 2048
    w = nv().quantize(to_gpu(workloads.weight(201, 1, N, K)))
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    _fill(x, 299, M, K)
    a = nv().quantize(x, "per_row")
    y = nv().gemm(a, w, torch.float32)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv().quantize(x, "per_row", out=a)
        nv().gemm(a, w, torch.float32, out=y)

    def eager():
        ae = nv().quantize(x, "per_row")
        return ae.codes, ae.global_scale, nv().gemm(ae, w, torch.float32)

    _replay_and_compare(g, x, M, K, (a.codes, a.global_scale, y), eager)


def test_graph_decode_balanced_rows():
    # N past one round of 32-row workgroups (8192 on 256 CUs): the balanced decode kernel,
    # with its shared LDS ring and per-step barriers, under capture.
    M, N, K = 8, 9000, 1024
    w = nv().quantize(to_gpu(workloads.weight(203, 1, N, K)))
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    _fill(x, 299, M, K)
    a = nv().quantize(x, "per_row")
    y = nv().gemm(a, w, torch.bfloat16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv().quantize(x, "per_row", out=a)
        nv().gemm(a, w, torch.bfloat16, out=y)

    def eager():
        ae = nv().quantize(x, "per_row")
        return ae.codes, ae.global_scale, nv().gemm(ae, w, torch.bfloat16)

    _replay_and_compare(g, x, M, K, (a.codes, a.global_scale, y), eager)


@pytest.mark.parametrize("M,F,K,mode", [(8, 4608, 1024, "per_row"), (300, 1024, 512, "per_tensor")])
def test_graph_mlp_swiglu_then_down(M, F, K, mode):
    # The gated MLP under capture: quantize the tokens, the fused gate+up GEMM with its SwiGLU
    # epilogue (h as bf16 and as NVFP4), then the down projection on the NVFP4 h.  Decode shape:
    # the balanced kernel with 64-row workgroups; prefill shape: the tile kernel.
    gate = nv().quantize(to_gpu(workloads.weight(204, 1, F, K)))
    up = nv().quantize(to_gpu(workloads.weight(204, 2, F, K)))
    down = nv().quantize(to_gpu(workloads.weight(204, 3, K, F)))
    wc, ws = nv().interleave_gate_up(gate, up)
    wg = torch.cat([gate.global_scale, up.global_scale])
    hg = torch.tensor([0.01], dtype=torch.float32, device=DEV)
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    _fill(x, 299, M, K)
    a = nv().quantize(x, mode)
    h, q = nv().gemm_swiglu(a, wc, ws, wg, torch.bfloat16, hg)
    y = nv().gemm(q, down, torch.bfloat16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv().quantize(x, mode, out=a)
        nv().gemm_swiglu(a, wc, ws, wg, torch.bfloat16, hg, out=h, q_out=q)
        nv().gemm(q, down, torch.bfloat16, out=y)

    def eager():
        ae = nv().quantize(x, mode)
        he, qe = nv().gemm_swiglu(ae, wc, ws, wg, torch.bfloat16, hg)
        return he, qe.codes, qe.scales, nv().gemm(qe, down, torch.bfloat16)

    _replay_and_compare(g, x, M, K, (h, q.codes, q.scales, y), eager)


def test_graph_fp8_kv_and_mxfp4():
    M, N, K = 256, 512, 512
    scale = torch.tensor([0.05], dtype=torch.float32, device=DEV)
    w = nv().to_mxfp4(nv().quantize(to_gpu(workloads.weight(202, 1, N, K))))
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    _fill(x, 299, M, K)
    q = nv().fp8_kv_quantize(x, scale)
    back = nv().fp8_kv_dequantize(q, scale, torch.bfloat16)
    a = nv().quantize(x)
    am = nv().to_mxfp4(a)
    y = nv().mxfp4_gemm(am, w.codes, w.scales, (N,), w.global_scale, torch.float32)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv().fp8_kv_quantize(x, scale, out=q)
        nv().fp8_kv_dequantize(q, scale, torch.bfloat16, out=back)
        nv().quantize(x, out=a)
        nv().to_mxfp4(a, out=am)
        nv().mxfp4_gemm(am, w.codes, w.scales, (N,), w.global_scale, torch.float32, out=y)

    def eager():
        qe = nv().fp8_kv_quantize(x, scale)
        ae = nv().to_mxfp4(nv().quantize(x))
        return (qe, nv().fp8_kv_dequantize(qe, scale, torch.bfloat16), ae.codes, ae.scales,
                nv().mxfp4_gemm(ae, w.codes, w.scales, (N,), w.global_scale, torch.float32))

    _replay_and_compare(g, x, M, K, (q, back, am.codes, am.scales, y), eager)


@pytest.mark.parametrize("N,K", [(9000, 1024), (2048, 1024), (1000, 1280)])
def test_graph_mxfp4_decode(N, K):
    # The three MXFP4 decode kernels under capture: balanced rows (N > 32 x CUs), per-wavefront
    # LDS rings (K % 512 == 0), and streaming from registers (other K); per-token scales.
    M = 4
    w = nv().to_mxfp4(nv().quantize(to_gpu(workloads.weight(205, 1, N, K))))
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    _fill(x, 299, M, K)
    a = nv().quantize(x, "per_row")
    am = nv().to_mxfp4(a)
    y = nv().mxfp4_gemm(am, w.codes, w.scales, (N,), w.global_scale, torch.float32)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv().quantize(x, "per_row", out=a)
        nv().to_mxfp4(a, out=am)
        nv().mxfp4_gemm(am, w.codes, w.scales, (N,), w.global_scale, torch.float32, out=y)

    def eager():
        ae = nv().to_mxfp4(nv().quantize(x, "per_row"))
        return ae.codes, ae.scales, nv().mxfp4_gemm(ae, w.codes, w.scales, (N,), w.global_scale, torch.float32)

    _replay_and_compare(g, x, M, K, (am.codes, am.scales, y), eager)


def test_graph_batch1_decode():
    # Batch 1: the matrix-vector kernel as two calls, and the one-call entry point that quantizes
    # the token inside the GEMM launch, captured together.
    N, K = 3000, 4160
    w = nv().quantize(to_gpu(workloads.weight(204, 1, N, K)))
    x = torch.empty((1, K), dtype=torch.bfloat16, device=DEV)
    _fill(x, 299, 1, K)
    a = nv().quantize(x)
    y = nv().gemm(a, w, torch.float32)
    y1, a1 = nv().decode_linear(x, w, out_dtype=torch.float32)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv().quantize(x, out=a)
        nv().gemm(a, w, torch.float32, out=y)
        nv().decode_linear(x, w, out_dtype=torch.float32, out=y1, a_out=a1)

    def eager():
        ae = nv().quantize(x)
        ye = nv().gemm(ae, w, torch.float32)
        yf, af = nv().decode_linear(x, w, out_dtype=torch.float32)
        return ae.codes, ae.global_scale, ye, af.codes, af.scales, af.global_scale, yf

    _replay_and_compare(g, x, 1, K, (a.codes, a.global_scale, y, a1.codes, a1.scales, a1.global_scale, y1), eager)
