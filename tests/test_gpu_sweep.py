"""GPU parity on the full-model sweep workload: every linear GEMM of a synthetic 64-layer hybrid
(48 GDN + 16 attention layers, hidden 5120, MLP 17408) at M = 16384 prefill tokens.  One launch
of each kind is run: the GDN input projection (six segments, own global scales), the GDN output
projection, the fused attention q/k/v and the attention output, the fused MLP gate+up and the
MLP down projection.  Activations and weights are quantized on the GPU; sampled rows of both are
checked bit-exact against the oracle (per-tensor scale from the whole tensor's amax), then 64
sampled output rows of the (fused) GEMM against the oracle's GEMM on the same operands."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_gemm_close, assert_quant_equal, nv, to_gpu, to_host

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
