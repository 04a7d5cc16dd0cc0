"""GPU parity on the full-model sweep workload: every linear GEMM of a synthetic 64-layer hybrid
(48 GDN + 16 attention layers, hidden 5120, MLP 17408) at M = 16384 prefill tokens.  One launch
of each kind is run: the GDN input projection (six segments, own global scales), the GDN output
projection, the fused attention q/k/v and the attention output, the fused MLP gate+up and the
MLP down projection.  Activations and weights are quantized on the GPU; sampled rows of both are
checked bit-exact against the oracle (per-tensor scale from the whole tensor's amax), then 64
sampled output rows of the (fused) GEMM against the oracle's GEMM on the same operands.  The
MLP gate+up launch is also run with its SwiGLU epilogue, as the sweep's MLP chain runs it.  A
slow test then runs all 256 launches on the weights the benchmark draws, with sampled rows and
columns (its comment says why)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_gemm_close, assert_quant_equal, assert_swiglu_close, nv, to_gpu, to_host

pytestmark = pytest.mark.gpu

KINDS = ["gdn_in", "gdn_out", "attn_qkv", "attn_o", "mlp_gate_up", "mlp_down"]


def _quantized_sampled(t: np.ndarray, rows: np.ndarray, what: str):
    q = nv().quantize(to_gpu(t))
    got = to_host(q)
    sg = ref.global_scale(t, ref.PER_TENSOR)
    assert got.global_scale.view(np.uint32)[0] == sg.view(np.uint32)[0], what
    assert_quant_equal(got, ref.quantize(t[rows], ref.GIVEN, float(sg[0])), rows=rows, what=what)
    return q, got


@pytest.mark.parametrize("kind", KINDS)
def test_sweep_launch(kind):
    sw = workloads.SWEEP
    launches = workloads.sweep_launches(sw)
    idx = next(i for i, l in enumerate(launches) if l.kind == kind)
    L = launches[idx]
    rng = np.random.default_rng(1000 + idx)
    rows = np.sort(rng.choice(sw.M, 64, replace=False))
    a, oa = _quantized_sampled(sw.x(idx, L.K), rows, f"{kind} x")
    segs, osegs = [], []
    for s, n in enumerate(L.widths):
        w = sw.w(idx, s, n, L.K)
        q, oq = _quantized_sampled(w, np.sort(rng.choice(n, 32, replace=False)), f"{kind} w{s}")
        segs.append(q)
        osegs.append(oq)
        del w
    y = nv().gemm_fused_segments(a, torch.cat([q.codes for q in segs]), torch.cat([q.scales for q in segs]),
                                 L.widths, torch.cat([q.global_scale for q in segs]), torch.bfloat16)
    Y, T = ref.fused_segments(oa, osegs, rows)
    worst = assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], Y, T, f"{kind} {sw.M}x{L.N}x{L.K}")
    print(f"{kind}: M={sw.M} N={L.N} K={L.K} segments={len(L.widths)} max err/T {worst:.3g}")


def test_sweep_mlp_swiglu():
    # The MLP gate+up launch as the sweep's MLP chain runs it: the SwiGLU epilogue on the
    # interleaved weights, h as fp32 and as NVFP4 in one launch; 64 sampled rows of h against
    # the oracle, and their NVFP4 encoding bit-exact against the oracle's GIVEN-mode quantize of
    # the same launch's fp32 h.
    sw = workloads.SWEEP
    launches = workloads.sweep_launches(sw)
    idx = next(i for i, l in enumerate(launches) if l.kind == "mlp_gate_up")
    L = launches[idx]
    F = L.widths[0]
    rng = np.random.default_rng(2000 + idx)
    rows = np.sort(rng.choice(sw.M, 64, replace=False))
    a, oa = _quantized_sampled(sw.x(idx, L.K), rows, "mlp x")
    (g, og), (u, ou) = [_quantized_sampled(sw.w(idx, s, F, L.K), np.sort(rng.choice(F, 32, replace=False)),
                                           f"mlp w{s}") for s in range(2)]
    wc, ws = nv().interleave_gate_up(g, u)
    wg = torch.cat([g.global_scale, u.global_scale])
    H, yg, tg, yu, tu = ref.swiglu_mlp(oa, og, ou, rows)
    s_h = np.float32(np.max(np.abs(H)) / 2688.0)
    h, q = nv().gemm_swiglu(a, wc, ws, wg, torch.float32, torch.tensor([s_h], dtype=torch.float32, device=DEV))
    sel = torch.from_numpy(rows).to(DEV)
    worst = assert_swiglu_close(h[sel], H, yg, tg, yu, tu, f"swiglu {sw.M}x{2 * F}x{L.K}")
    want = ref.quantize(h[sel].cpu().numpy(), ref.GIVEN, float(s_h))
    assert np.array_equal(q.scales[sel].cpu().numpy(), want.scales)
    assert np.array_equal(q.codes[sel].cpu().numpy(), want.codes)
    print(f"mlp swiglu: M={sw.M} F={F} K={L.K} max err/bound {worst:.3g}")


def _oracle_sampled(t_host: np.ndarray, amax: float, rows: np.ndarray) -> ref.NVFP4:
    """The oracle's quantization of rows of a tensor under the tensor's per-tensor global scale
    (fl32(amax / 2688) from the exact max |x| of the whole tensor): the same bytes as quantizing
    the whole tensor, for the sampled rows."""
    sg = ref.global_scale(np.asarray([[amax]], np.float32), ref.PER_TENSOR)
    return ref.quantize(t_host[rows], ref.GIVEN, float(sg[0]))


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_sweep_every_launch_as_benchmarked():
    # All 256 launches of the sweep on the weights the benchmark itself draws (bench.py's seeded
    # torch generator) and its three activations (one per K): per launch, 64 sampled rows of the
    # activation and 256 sampled rows of the weight (every row of the 48-wide gate segments, the
    # rest spread over the segments) are quantized by the oracle from the same bf16 values under
    # the tensors' own global scales and compared bit for bit with the GPU's bytes; then the GPU's
    # fused GEMM output at those 64 rows x sampled columns is compared with the oracle's GEMM of its
    # own quantized operands, within 1e-4 * sum |a w| plus half a bf16 ulp.  Columns are sampled
    # because the oracle's full-width GEMM over all 256 launches would dequantize 22.8 G weights.
    import bench
    sw = workloads.SWEEP
    launches = workloads.sweep_launches(sw)
    rng = np.random.default_rng(4242)
    acts = {}
    for K in sorted({L.K for L in launches}):
        x = sw.x(0, K)
        rows = np.sort(rng.choice(sw.M, 64, replace=False))
        a = nv().quantize(to_gpu(x))
        oa = _oracle_sampled(x, float(np.abs(x).max()), rows)
        assert_quant_equal(to_host(a), oa, rows=rows, what=f"x K={K}")
        assert a.global_scale.cpu().numpy().view(np.uint32)[0] == oa.global_scale.view(np.uint32)[0], f"x K={K}"
        acts[K] = (a, oa, rows)
        del x
    worst = 0.0
    for li, L, segs in bench.sweep_weight_draws(sw, launches, DEV):
        a, oa, rows = acts[L.K]
        qs, cols, osegs = [], [], []
        off = 0
        per = max(1, 256 // len(L.widths))
        for s, (w, n) in enumerate(zip(segs, L.widths)):
            q = nv().quantize(w)
            pick = np.arange(n) if n <= per else np.sort(rng.choice(n, per, replace=False))
            w_rows = w[torch.from_numpy(pick).to(DEV)].float().cpu().numpy()
            amax = float(w.abs().max().float().item())
            o = _oracle_sampled(w_rows, amax, np.arange(len(pick)))
            sel = torch.from_numpy(pick).to(DEV)
            assert np.array_equal(q.codes[sel].cpu().numpy(), o.codes) and \
                np.array_equal(q.scales[sel].cpu().numpy(), o.scales), f"launch {li} ({L.kind}) segment {s}: bytes differ"
            assert q.global_scale.cpu().numpy().view(np.uint32)[0] == o.global_scale.view(np.uint32)[0], \
                f"launch {li} w{s}"
            qs.append(q)
            osegs.append(o)
            cols.append(off + pick)
            off += n
        del segs
        y = nv().gemm_fused_segments(a, torch.cat([q.codes for q in qs]), torch.cat([q.scales for q in qs]),
                                     L.widths, torch.cat([q.global_scale for q in qs]), torch.bfloat16)
        Y, T = ref.fused_segments(oa, osegs)          # oa holds the 64 sampled rows only
        cols = np.concatenate(cols)
        got_y = y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)]
        worst = max(worst, assert_gemm_close(got_y, Y, T, f"launch {li} ({L.kind}) {sw.M}x{L.N}x{L.K}"))
        del y, qs
        if li % 32 == 0:
            print(f"sweep launch {li}/{len(launches)} ok, max err/T so far {worst:.3g}", flush=True)
    print(f"all {len(launches)} sweep launches: max err/T {worst:.3g}")
