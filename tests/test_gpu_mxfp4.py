"""GPU parity of the lossy NVFP4 -> MXFP4 variant against the oracle: nvfp4_to_mxfp4 bit-exact
(codes and E8M0 bytes, in place too, zero blocks included), and nvfp4_mxfp4_gemm within
1e-4 * sum_k |a_k w_k| (plus half a bf16 ulp for bf16 output) of the oracle's MXFP4 GEMM on
the same operands: tile-aligned and ragged shapes, small M (the decode kernel, up to the MLP's
full up and down shapes), fused segments, per-row activation scales, and the full prefill shape
on sampled rows.  The error of the variant
against the exact NVFP4 product is measured and must stay within the range the re-encoding
allows (it is lossy by design; the figure is reported, not a parity claim)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_gemm_close, assert_quant_equal, nv, to_gpu

pytestmark = pytest.mark.gpu


def _mx_equal(got, want: ref.MXFP4, what: str = "") -> None:
    gc, gs = got.codes.cpu().numpy(), got.scales.cpu().numpy()
    assert gs.shape == want.scales.shape and gc.shape == want.codes.shape, what
    bad = np.argwhere(gs != want.scales)
    assert bad.size == 0, f"{what}: {len(bad)} E8M0 bytes differ, first {bad[:3].tolist()}"
    bad = np.argwhere(gc != want.codes)
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first {bad[:3].tolist()}"


def _quant(x, mode="per_tensor"):
    xg = to_gpu(x)
    q = nv().quantize(xg, mode)
    o = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW if mode == "per_row" else ref.PER_TENSOR)
    assert_quant_equal(q, o, what="nvfp4")
    return q, o


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (64, 512), (300, 5120)])
def test_reencode_bit_exact(rows, cols):
    x = workloads.activation(80 + rows, 0, rows, cols, outlier_frac=0.01, outlier_gain=50.0)
    x[:, :32] = 0.0                     # an all-zero block in every row
    if rows > 2:
        x[1] = 0.0                      # an all-zero row
    q, o = _quant(x)
    m = nv().to_mxfp4(q)
    torch.cuda.synchronize()
    _mx_equal(m, ref.mxfp4_from_nvfp4(o), f"{rows}x{cols}")


def test_reencode_in_place_and_weights():
    w = workloads.weight(90, 1, 512, 1024, sigma=0.02)
    q, o = _quant(w)
    want = ref.mxfp4_from_nvfp4(o)
    out = nv().MXFP4Tensor(q.codes, torch.empty((512, 1024 // 32), dtype=torch.uint8, device=DEV), q.global_scale)
    nv().to_mxfp4(q, out=out)           # codes overwritten in place
    torch.cuda.synchronize()
    _mx_equal(out, want, "in place")


def _mx_pair(M, N, K, seed, a_mode="per_tensor"):
    qa, oa = _quant(workloads.activation(seed, 0, M, K, outlier_frac=0.001, outlier_gain=50.0), a_mode)
    qw, ow = _quant(workloads.weight(seed, 1, N, K, sigma=0.02))
    ma, mw = nv().to_mxfp4(qa), nv().to_mxfp4(qw)
    oma, omw = ref.mxfp4_from_nvfp4(oa), ref.mxfp4_from_nvfp4(ow)
    _mx_equal(ma, oma, "A")
    _mx_equal(mw, omw, "W")
    return ma, mw, oma, omw, oa, ow


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 416, 512), (257, 1000, 768), (64, 96, 256),
                                   (16, 512, 512), (1, 256, 256), (5, 130, 1024)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_mx_gemm(M, N, K, out_dtype):
    ma, mw, oma, omw, _, _ = _mx_pair(M, N, K, seed=100 + M + N)
    y = nv().mxfp4_gemm(ma, mw.codes, mw.scales, (N,), mw.global_scale, out_dtype)
    Y, T = ref.mx_gemm(oma, omw)
    assert_gemm_close(y, Y, T, f"mx {M}x{N}x{K} {out_dtype}")


def test_mx_gemm_per_row_scales_and_segments():
    M, K, widths = 200, 512, (128, 48, 48, 96)
    qa, oa = _quant(workloads.activation(110, 0, M, K, outlier_frac=0.001, outlier_gain=50.0), "per_row")
    ma, oma = nv().to_mxfp4(qa), ref.mxfp4_from_nvfp4(oa)
    _mx_equal(ma, oma, "A")
    segs, osegs = [], []
    for i, n in enumerate(widths):
        q, o = _quant(workloads.weight(110, 1 + i, n, K, sigma=0.02 * (i + 1)))
        segs.append(nv().to_mxfp4(q))
        osegs.append(ref.mxfp4_from_nvfp4(o))
    y = nv().mxfp4_gemm(ma, torch.cat([s.codes for s in segs]), torch.cat([s.scales for s in segs]), widths,
                        torch.cat([s.global_scale for s in segs]), torch.float32)
    ys, ts = zip(*(ref.mx_gemm(oma, o) for o in osegs))
    assert_gemm_close(y, np.concatenate(ys, axis=1), np.concatenate(ts, axis=1), "mx fused per-row")


def _random_mx(g, R, K, per_row=False):
    """Seeded MXFP4 bytes: random codes, E8M0 scales over 2^-9 .. 2^8, global scale per row or
    per tensor."""
    codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = g.integers(118, 136, (R, K // 32), dtype=np.uint8)
    gs = g.uniform(0.5, 2.0, R if per_row else 1).astype(np.float32)
    return ref.MXFP4(codes, scales, gs, R, K)


def _mx_device(o: ref.MXFP4):
    return nv().MXFP4Tensor(torch.from_numpy(o.codes).to(DEV), torch.from_numpy(o.scales).to(DEV),
                            torch.from_numpy(np.asarray(o.global_scale, np.float32)).to(DEV))


# M <= 16: the MXFP4 decode kernels.  K % 512 == 0: the balanced kernel when N > 32 x CUs (two
# or three 32-row groups per workgroup, 8 wavefronts on one ring), else per-wavefront LDS rings
# (16 to 32 W rows per workgroup, stage pairs split over 4 wavefronts); other K: from registers.
@pytest.mark.parametrize("M,N,K", [(1, 17408, 5120), (16, 17408, 5120),   # MLP up: balanced, 3 groups
                                   (4, 9000, 1024),     # balanced, 2 groups
                                   (9, 30000, 512),     # balanced, 2 rounds; one stage pair
                                   (16, 16700, 10240),  # balanced, 3 groups; last workgroup 2 rows
                                   (2, 12000, 14336),   # balanced, 2 groups: K too long for 3
                                   (16, 5120, 17408),   # MLP down: per-wavefront rings
                                   (7, 2000, 1536),     # 16-row workgroups, 3 stage pairs over 4 wavefronts
                                   (3, 640, 32768),     # 32 stages per wavefront: two scale blocks each
                                   (8, 1000, 1280),     # registers: 5 stages over 4 wavefronts
                                   (2, 64, 256),        # registers: one stage, three wavefronts idle
                                   (11, 4128, 2304)])
def test_mx_decode(M, N, K):
    g = np.random.default_rng(M * 7919 + N + K)
    oa, ow = _random_mx(g, M, K, per_row=True), _random_mx(g, N, K)
    w = _mx_device(ow)
    for out_dtype in (torch.float32, torch.bfloat16):
        y = nv().mxfp4_gemm(_mx_device(oa), w.codes, w.scales, (N,), w.global_scale, out_dtype)
        Y, T = ref.mx_gemm(oa, ow)
        assert_gemm_close(y, Y, T, f"mx decode {M}x{N}x{K} {out_dtype}")


@pytest.mark.parametrize("K,widths", [(768, (96, 48, 48, 40)), (1024, (96, 48, 48, 40)), (1024, (5000, 48, 4000))])
def test_mx_decode_segments(K, widths):
    M = 4
    g = np.random.default_rng(17)
    oa = _random_mx(g, M, K, per_row=True)
    segs = [_random_mx(g, n, K) for n in widths]
    ds = [_mx_device(o) for o in segs]
    y = nv().mxfp4_gemm(_mx_device(oa), torch.cat([d.codes for d in ds]), torch.cat([d.scales for d in ds]), widths,
                        torch.cat([d.global_scale for d in ds]), torch.float32)
    ys, ts = zip(*(ref.mx_gemm(oa, o) for o in segs))
    assert_gemm_close(y, np.concatenate(ys, axis=1), np.concatenate(ts, axis=1), "mx decode segments")


def test_mx_gemm_full_prefill_shape_sampled_rows():
    p = workloads.PREFILL
    qa, oa = _quant(p.x())
    qw, ow = _quant(p.w())
    ma, mw = nv().to_mxfp4(qa), nv().to_mxfp4(qw)
    oma, omw = ref.mxfp4_from_nvfp4(oa), ref.mxfp4_from_nvfp4(ow)
    _mx_equal(ma, oma, "A")
    _mx_equal(mw, omw, "W")
    y = nv().mxfp4_gemm(ma, mw.codes, mw.scales, (p.N,), mw.global_scale, torch.bfloat16)
    rows = np.concatenate([[0, p.M - 1], np.random.default_rng(11).choice(p.M, 30, replace=False)])
    Y, T = ref.mx_gemm(oma, omw, rows)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], Y, T, "mx prefill")
    # The variant's error against the exact NVFP4 product on the same rows (lossy by design).
    Yn, _ = ref.gemm(oa, ow, rows)
    rel = float(np.linalg.norm(Y - Yn) / np.linalg.norm(Yn))
    print(f"MXFP4 re-encoding: relative RMS error vs the NVFP4 GEMM = {rel:.4f}")
    assert 0.01 < rel < 0.25
