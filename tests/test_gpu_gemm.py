"""GPU parity of nvfp4_gemm and nvfp4_gemm_fused_segments against the oracle:
per-element |y - Y| <= 1e-4 * sum_k |a_k w_k| (plus half a bf16 ulp for bf16 output), an
integer-exact special case compared bitwise, fused == separate, and the global-scale
mismatch reproduced as a negative control."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_gemm_close, assert_quant_equal, nv, to_device, to_gpu, to_host

pytestmark = pytest.mark.gpu


def _quant_pair(x, w, a_mode="per_tensor", bf16=True):
    """Quantize on the GPU, check bit-exactness, return (gpu A, gpu W, oracle A, oracle W)."""
    xg, wg = to_gpu(x, bf16), to_gpu(w, bf16)
    a, q = nv().quantize(xg, a_mode), nv().quantize(wg)
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW if a_mode == "per_row" else ref.PER_TENSOR)
    ow = ref.quantize(wg.float().cpu().numpy())
    assert_quant_equal(a, oa, what="A")
    assert_quant_equal(q, ow, what="W")
    return a, q, oa, ow


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny(out_dtype):
    t = workloads.TINY
    a, w, oa, ow = _quant_pair(t.x(), t.w(), bf16=False)
    y = nv().gemm(a, w, out_dtype)
    Y, T = ref.gemm(oa, ow)
    assert_gemm_close(y, Y, T, "tiny")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prefill_sampled_rows(out_dtype):
    p = workloads.PREFILL
    a, w, oa, ow = _quant_pair(p.x(), p.w())
    y = nv().gemm(a, w, out_dtype)
    rows = np.sort(np.random.default_rng(1).choice(p.M, 48, replace=False))
    rows = np.concatenate([[0, p.M - 1], rows])
    Y, T = ref.gemm(oa, ow, rows)
    worst = assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], Y, T, "prefill")
    print(f"prefill max err/T = {worst:.3g}")


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("a_mode", ["per_row", "per_tensor"])
def test_decode(M, a_mode):
    d = workloads.DECODE
    a, w, oa, ow = _quant_pair(d.x(M), d.w(), a_mode)
    y = nv().gemm(a, w, torch.bfloat16)
    Y, T = ref.gemm(oa, ow)
    assert_gemm_close(y, Y, T, f"decode M={M}")


def _raw_values(t):
    """E2M1(code) * E4M3(scale) per element, without the global scale (exact in binary32)."""
    v = ref.e2m1_decode(ref.unpack_codes(t.codes)).astype(np.float32)
    return v * np.repeat(ref.e4m3_decode(t.scales).astype(np.float32), 16, axis=1)


# Decode where the kernels' fp32 accumulation rounds: 1 % of the token's channels x50 and weight
# blocks scaled by 2^((k / 16) mod 7), so the block scales of a row span six binades more than the
# Gaussian cases, where every partial sum is exactly representable in fp32.  The shapes reach the
# 4 x 4 x 4 kernel (M <= 4, five and four row groups on 256 CUs) and the 16 x 16 x 32 K-split
# kernel copying one token chunk (M = 6, 8) and two (M = 16).
@pytest.mark.parametrize("M,N,K", [(4, 5120, 17408), (3, 4700, 4096), (8, 6000, 2560), (6, 8000, 1280),
                                   (16, 5120, 4096)])
def test_decode_inexact_accumulation(M, N, K):
    x = workloads.activation(77, M, M, K, outlier_frac=0.01)
    gain = np.exp2((np.arange(K) // 16) % 7).astype(np.float32)
    w = workloads.weight(77, 1, N, K) * gain[None, :]
    a, q, oa, ow = _quant_pair(x, w, "per_row")
    # Precondition, on the host: a sequential fp32 sum of these operands differs from the exact
    # sum somewhere, so exactness of the accumulation cannot hide an ordering or reduction error.
    ra, rw = _raw_values(oa), _raw_values(ow)
    cols = np.arange(0, N, max(1, N // 64))
    acc = np.zeros((M, cols.size), np.float32)
    for k in range(K):
        acc += ra[:, k:k + 1] * rw[cols, k][None, :]
    exact = ra.astype(np.float64) @ rw[cols].astype(np.float64).T
    assert np.any(acc.astype(np.float64) != exact), "the fp32 accumulation is exact for these operands"
    for out_dtype in (torch.float32, torch.bfloat16):
        y = nv().gemm(a, q, out_dtype)
        Y, T = ref.gemm(oa, ow)
        assert_gemm_close(y, Y, T, f"inexact decode M={M} N={N} K={K} {out_dtype}")


@pytest.fixture(scope="module")
def decode_up_weight():
    """The MLP up projection's weight at decode (17408 x 5120), quantized on the GPU and by the
    oracle once for the module."""
    wg = to_gpu(workloads.DECODE_UP.w())
    q = nv().quantize(wg)
    ow = ref.quantize(wg.float().cpu().numpy())
    assert_quant_equal(q, ow, what="W")
    return q, ow


@pytest.mark.parametrize("M", [1, 16])
def test_decode_up_projection(M, decode_up_weight):
    # The balanced decode kernel at its full shape: 68 W rows per workgroup, one round.
    q, ow = decode_up_weight
    xg = to_gpu(workloads.DECODE_UP.x(M))
    a = nv().quantize(xg, "per_row")
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW)
    assert_quant_equal(a, oa, what="A")
    Y, T = ref.gemm(oa, ow)
    assert_gemm_close(nv().gemm(a, q, torch.bfloat16), Y, T, f"decode up M={M}")


def _fused_weights(f, K=None, rows=None):
    segs_gpu, segs_ora = [], []
    for i in range(len(f.widths)):
        wg = to_gpu(f.w(i))
        q = nv().quantize(wg)
        o = ref.quantize(wg.float().cpu().numpy())
        assert_quant_equal(q, o, what=f"w{i}")
        segs_gpu.append(q)
        segs_ora.append(o)
    codes = torch.cat([q.codes for q in segs_gpu])
    scales = torch.cat([q.scales for q in segs_gpu])
    globals_ = torch.cat([q.global_scale for q in segs_gpu])
    return segs_gpu, segs_ora, codes, scales, globals_


def test_fused_gdn_projections():
    f = workloads.FUSED
    xg = to_gpu(f.x())
    a = nv().quantize(xg)
    oa = ref.quantize(xg.float().cpu().numpy())
    assert_quant_equal(a, oa, what="x")
    segs_gpu, segs_ora, codes, scales, globals_ = _fused_weights(f)
    y = nv().gemm_fused_segments(a, codes, scales, f.widths, globals_, torch.bfloat16)
    rows = np.concatenate([[0, f.M - 1], np.random.default_rng(3).choice(f.M, 30, replace=False)])
    Y, T = ref.fused_segments(oa, segs_ora, rows)
    assert_gemm_close(y[torch.from_numpy(rows).to(DEV)], Y, T, "fused")
    # fused == six separate launches, bitwise (same kernel, same K order per element)
    off = 0
    for q, n in zip(segs_gpu, f.widths):
        ys = nv().gemm(a, q, torch.bfloat16)
        assert torch.equal(ys, y[:, off:off + n]), f"segment at {off}"
        off += n


def test_shared_global_scale_reproduces_the_mismatch():
    # A fused launch that applies the first module's global scale to every segment scales
    # segment i by s_g0 / s_gi: the global-scale mismatch (repaired by per-segment scales).
    f = workloads.FUSED
    xg = to_gpu(f.x(256))
    a = nv().quantize(xg)
    segs_gpu, segs_ora, codes, scales, globals_ = _fused_weights(f)
    good = nv().gemm_fused_segments(a, codes, scales, f.widths, globals_, torch.float32)
    bad = nv().gemm_fused_segments(a, codes, scales, f.widths, globals_[:1].repeat(len(f.widths)),
                                   torch.float32)
    off = 0
    g0 = globals_[0].item()
    for i, n in enumerate(f.widths):
        ratio = g0 / globals_[i].item()
        gs, bs = good[:, off:off + n].double(), bad[:, off:off + n].double()
        assert torch.allclose(bs, gs * ratio, rtol=1e-6, atol=1e-30 + 1e-6 * gs.abs().max().item() * ratio)
        off += n
    # the gate segments (sigma 0.05) come out at less than half their true size
    assert g0 / globals_[4].item() < 0.5


def _unit_scale(codes_np):
    R, C = codes_np.shape
    return ref.NVFP4(ref.pack_codes(codes_np), np.full((R, C // 16), 0x38, np.uint8), np.ones(1, np.float32), R, C)


@pytest.mark.parametrize("M,N,K", [(4096, 17408, 5120), (16, 5120, 17408), (1, 5120, 17408), (8192, 12384, 5120),
                                   (300, 200, 384)])
def test_integer_exact_special_case(M, N, K):
    # Scale bytes 0x38 (1.0) and global scales 1.0: Y = integer matmul / 4, exact in fp32 in
    # any summation order, so the GPU must match int64 arithmetic bit for bit.
    g = np.random.default_rng(M + N + K)
    ca = g.integers(0, 16, (M, K), dtype=np.uint8)
    cw = g.integers(0, 16, (N, K), dtype=np.uint8)
    y = nv().gemm(to_device(_unit_scale(ca)), to_device(_unit_scale(cw)), torch.float32)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)
    rows = np.arange(M) if M <= 64 else np.sort(g.choice(M, 64, replace=False))
    ia = (np.where(ca[rows] & 8, -1, 1) * twice[ca[rows] & 7]).astype(np.float64)
    iw = (np.where(cw & 8, -1, 1) * twice[cw & 7]).astype(np.float64)
    want = (ia @ iw.T) / 4.0          # integers below 2^53: exact in float64 BLAS
    got = y[torch.from_numpy(rows).to(DEV)].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M,N,K", [(17, 50, 128), (37, 300, 384), (300, 1, 256), (257, 257, 128),
                                   (5, 33, 272), (40, 24, 16), (2, 7, 4112)])
@pytest.mark.parametrize("a_mode", ["per_tensor", "per_row"])
def test_ragged_shapes(M, N, K, a_mode):
    x = workloads.activation(31, M, M, K, outlier_frac=0.02)
    w = workloads.weight(31, 1000 + N, N, K)
    a, q, oa, ow = _quant_pair(x, w, a_mode)
    for dt in (torch.float32, torch.bfloat16):
        y = nv().gemm(a, q, dt)
        Y, T = ref.gemm(oa, ow)
        assert_gemm_close(y, Y, T, f"{M}x{N}x{K} {a_mode} {dt}")


# Decode path (M <= 16, K a multiple of 128): odd chunk counts (a last 128-wide chunk after
# the 256-wide stages; K = 128 has no stage at all), per-wave stage splits of unequal length,
# N not a multiple of the workgroup's rows (17 and 32 rows per workgroup for N = 4100 and
# 7990 on 256 CUs, a last workgroup of 3 and 22 rows), N = 1.
@pytest.mark.parametrize("M,N,K", [(3, 100, 384), (16, 33, 128), (7, 1, 640), (1, 4097, 1152),
                                   (16, 64, 2048), (2, 96, 2304), (16, 200, 4224), (4, 4100, 512),
                                   (11, 7990, 1024)])
@pytest.mark.parametrize("a_mode", ["per_tensor", "per_row"])
def test_decode_ragged(M, N, K, a_mode):
    x = workloads.activation(33, M, M, K, outlier_frac=0.02)
    w = workloads.weight(33, 2000 + N, N, K)
    a, q, oa, ow = _quant_pair(x, w, a_mode)
    Y, T = ref.gemm(oa, ow)
    for dt in (torch.float32, torch.bfloat16):
        y = nv().gemm(a, q, dt)
        assert_gemm_close(y, Y, T, f"decode {M}x{N}x{K} {a_mode} {dt}")


# Balanced decode kernel (M <= 16, K a multiple of 256, N past one round of 32-row workgroups,
# 8192 on 256 CUs): rows per workgroup chosen so that the grid is a whole number of rounds over
# the CUs.  Shapes hit 3 to 5 row groups per workgroup, partial last groups and chunks, one or
# two token chunks, two rounds, fewer stages than the copy ring holds, scale blocks cut short,
# and the LDS limit (K = 10240 still fits five row groups, 10496 goes to the other kernel);
# below the cut, the K-split kernel.
@pytest.mark.parametrize("M,N,K", [(1, 8455, 256), (5, 8455, 512), (16, 12384, 1792), (9, 17408, 2304),
                                   (16, 20481, 768), (8, 16700, 10240), (1, 16700, 10496), (3, 5120, 8448),
                                   (2, 5120, 17408), (16, 300, 1280)])
def test_decode_balanced_rows(M, N, K):
    # Seeded NVFP4 operands built directly (random codes, block scales over 2^-5 .. 2^1, a
    # global scale per token row), the same bytes for the GPU and the oracle.
    g = np.random.default_rng(M * N + K)

    def operand(R, per_row):
        codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
        scales = g.integers(0x10, 0x40, (R, K // 16), dtype=np.uint8)
        gs = g.uniform(0.5, 2.0, R if per_row else 1).astype(np.float32)
        return ref.NVFP4(codes, scales, gs, R, K)

    oa, ow = operand(M, True), operand(N, False)
    Y, T = ref.gemm(oa, ow)
    y = nv().gemm(to_device(oa), to_device(ow), torch.float32)
    assert_gemm_close(y, Y, T, f"decode {M}x{N}x{K}")


# Batch-1 decode (M = 1, K a multiple of 64, N up to one round of 32-row workgroups or K not a
# multiple of 256) runs the matrix-vector kernel: a workgroup of 16 wavefronts per CU, each W row
# cut into 2048-value items, the workgroup's items shared out in 16 equal ranges.  Shapes: one group of 32 values (K = 64, one short item), K not a multiple of
# 128, items per row of 1, 3 and 16 (the token's copies then outnumber the wavefronts), N = 1
# and 7 (wavefronts with no items, rows cut over many wavefronts), ragged last workgroups, and a
# row count whose LDS slots no longer fit (N = 400003 at K = 64: the MFMA decode kernel).
@pytest.mark.parametrize("N,K", [(1, 64), (7, 320), (300, 4160), (600, 32768), (70001, 128), (5120, 6208),
                                 (400003, 64)])
def test_gemv_batch1(N, K):
    g = np.random.default_rng(N + K)

    def operand(R):
        codes = g.integers(0, 256, (R, K // 2), dtype=np.uint8)
        scales = g.integers(0x10, 0x40, (R, K // 16), dtype=np.uint8)
        gs = g.uniform(0.5, 2.0, 1).astype(np.float32)
        return ref.NVFP4(codes, scales, gs, R, K)

    oa, ow = operand(1), operand(N)
    Y, T = ref.gemm(oa, ow)
    a, w = to_device(oa), to_device(ow)
    for dt in (torch.float32, torch.bfloat16):
        assert_gemm_close(nv().gemm(a, w, dt), Y, T, f"gemv 1x{N}x{K} {dt}")


def test_gemv_batch1_segments_and_pitch():
    # Fused segments with their own global scales, and an output row pitch past N.
    K, widths = 1088, (40, 8, 1000)
    xg = to_gpu(workloads.activation(37, 0, 1, K))
    a = nv().quantize(xg, "per_row")
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW)
    gq, oq = [], []
    for i, n in enumerate(widths):
        wg = to_gpu(workloads.weight(37, 10 + i, n, K, sigma=0.02 * (i + 1)))
        gq.append(nv().quantize(wg))
        oq.append(ref.quantize(wg.float().cpu().numpy()))
    y = nv().gemm_fused_segments(a, torch.cat([q.codes for q in gq]), torch.cat([q.scales for q in gq]), widths,
                                 torch.cat([q.global_scale for q in gq]), torch.float32)
    Y, T = ref.fused_segments(oa, oq)
    assert_gemm_close(y, Y, T, "gemv fused")
    Y2, T2 = ref.gemm(oa, oq[2])
    for dt in (torch.float32, torch.bfloat16):
        big = torch.full((1, 2000), 7.0, dtype=dt, device=DEV)
        nv().gemm(a, gq[2], dt, out=big[:, :1000])
        assert_gemm_close(big[:, :1000], Y2, T2, f"gemv pitch {dt}")
        assert torch.all(big[:, 1000:] == 7.0)


def test_decode_balanced_rows_segments():
    M, K, widths = 4, 2048, (4000, 48, 3000)
    xg = to_gpu(workloads.activation(36, 0, M, K))
    a = nv().quantize(xg, "per_row")
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW)
    gq, oq = [], []
    for i, n in enumerate(widths):
        wg = to_gpu(workloads.weight(36, 10 + i, n, K, sigma=0.02 * (i + 1)))
        gq.append(nv().quantize(wg))
        oq.append(ref.quantize(wg.float().cpu().numpy()))
    y = nv().gemm_fused_segments(a, torch.cat([q.codes for q in gq]), torch.cat([q.scales for q in gq]), widths,
                                 torch.cat([q.global_scale for q in gq]), torch.bfloat16)
    Y, T = ref.fused_segments(oa, oq)
    assert_gemm_close(y, Y, T, "decode fused, balanced rows")


def test_decode_fused_segments():
    M, K, widths = 4, 640, (40, 8, 100)
    xg = to_gpu(workloads.activation(34, 0, M, K))
    a = nv().quantize(xg, "per_row")
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW)
    gq, oq = [], []
    for i, n in enumerate(widths):
        wg = to_gpu(workloads.weight(34, 10 + i, n, K, sigma=0.02 * (i + 1)))
        gq.append(nv().quantize(wg))
        oq.append(ref.quantize(wg.float().cpu().numpy()))
    y = nv().gemm_fused_segments(a, torch.cat([q.codes for q in gq]), torch.cat([q.scales for q in gq]), widths,
                                 torch.cat([q.global_scale for q in gq]), torch.float32)
    Y, T = ref.fused_segments(oa, oq)
    assert_gemm_close(y, Y, T, "decode fused")


@pytest.mark.parametrize("M", [1, 4])
def test_long_k_at_decode(M):
    """K = 2^24 with few tokens: the tiled and decode kernels address rows with 32-bit offsets
    that are only guaranteed below 2^24, so these shapes run the plain kernel."""
    K, N = 1 << 24, 3
    rng = np.random.default_rng(24 + M)
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    a, q, oa, ow = _quant_pair(x, w)
    y = nv().gemm(a, q, torch.float32)
    Y, T = ref.gemm(oa, ow)
    assert_gemm_close(y, Y, T, f"K = 2^24, M = {M}")


def test_decode_deterministic():
    d = workloads.DECODE
    a, w, _, _ = _quant_pair(d.x(16), d.w()[:512])
    assert torch.equal(nv().gemm(a, w), nv().gemm(a, w))


def test_output_row_pitch():
    x = workloads.activation(32, 0, 40, 256)
    w = workloads.weight(32, 1, 96, 256)
    a, q, oa, ow = _quant_pair(x, w)
    big = torch.full((40, 128), 7.0, dtype=torch.float32, device=DEV)
    nv().gemm(a, q, torch.float32, out=big[:, :96])
    Y, T = ref.gemm(oa, ow)
    assert_gemm_close(big[:, :96], Y, T, "pitched")
    assert (big[:, 96:] == 7.0).all()


def test_empty_products():
    a = nv().quantize(torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV), "per_row")
    w = nv().quantize(torch.ones((8, 128), dtype=torch.bfloat16, device=DEV))
    assert nv().gemm(a, w).shape == (0, 8)


def test_deterministic():
    p = workloads.PREFILL
    a, w, _, _ = _quant_pair(p.x(512), p.w()[:1024])
    assert torch.equal(nv().gemm(a, w), nv().gemm(a, w))


def test_batch1_per_row_flag_at_the_abi():
    # One token: a per-row global scale and a per-tensor one are the same number, and the C ABI
    # accepts either flag; both calls must give the same bits (the binding always passes 0 here).
    N, K = 3000, 2048
    g = np.random.default_rng(5)
    ow = ref.NVFP4(g.integers(0, 256, (N, K // 2), dtype=np.uint8), g.integers(0x10, 0x40, (N, K // 16), dtype=np.uint8),
                   np.array([0.75], np.float32), N, K)
    oa = ref.NVFP4(g.integers(0, 256, (1, K // 2), dtype=np.uint8), g.integers(0x10, 0x40, (1, K // 16), dtype=np.uint8),
                   np.array([1.25], np.float32), 1, K)
    a, w = to_device(oa), to_device(ow)
    ys = []
    for per_row in (0, 1):
        y = torch.empty((1, N), dtype=torch.float32, device=DEV)
        st = nv().lib.nvfp4_gemm(1, N, K, a.codes.data_ptr(), a.scales.data_ptr(), a.global_scale.data_ptr(), per_row,
                                 w.codes.data_ptr(), w.scales.data_ptr(), w.global_scale.data_ptr(), y.data_ptr(), 0, N,
                                 None, 0, torch.cuda.current_stream(DEV).cuda_stream)
        assert st == 0
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    Y, T = ref.gemm(oa, ow)
    assert_gemm_close(ys[0], Y, T, "batch-1 per-row flag")
