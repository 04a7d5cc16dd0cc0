"""GPU parity of nvfp4_quantize: codes, scale bytes and global scales bit-exact against the
oracle on every workload's tensors and on edge cases."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_quant_equal, nv, to_gpu, to_host

pytestmark = pytest.mark.gpu


def _check(x: np.ndarray, mode="per_tensor", bf16=True, given=None, what=""):
    xg = to_gpu(x, bf16)
    gs = None if given is None else torch.tensor([given], dtype=torch.float32, device=DEV)
    got = nv().quantize(xg, mode, gs)
    xs = xg.float().cpu().numpy()          # the exact values the GPU saw
    want = ref.quantize(xs, {"per_tensor": ref.PER_TENSOR, "per_row": ref.PER_ROW, "given": ref.GIVEN}[mode],
                        given)
    assert_quant_equal(got, want, what=what or mode)
    return got, want


def test_tiny_fp32_activations_and_weights():
    _check(workloads.TINY.x(), bf16=False, what="tiny x")
    _check(workloads.TINY.w(), bf16=False, what="tiny w")


def test_prefill_activations_full():
    _check(workloads.PREFILL.x(), what="prefill x 4096x5120")


def test_prefill_weights_full():
    _check(workloads.PREFILL.w(), what="prefill w 17408x5120")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_per_token_activations(M):
    x = workloads.DECODE.x(M)
    _check(x, "per_row", what=f"decode x M={M} per_row")
    _check(x, "per_tensor", what=f"decode x M={M} per_tensor")


# Per-row mode routes by the blocks per row (bpr) when rows are fewer than the CUs: 1024-thread
# workgroups holding one block per thread (bpr <= 1024) or two (<= 2048); past that the
# 256-thread kernel (bf16 up to 2048 blocks per row, fp32 up to 1024) or the row-scale +
# encode pair.  Each side of every boundary, both input types.
@pytest.mark.parametrize("bpr", [1024, 1025, 2048, 2049, 4100])
@pytest.mark.parametrize("bf16", [True, False])
def test_per_row_block_count_routes(bpr, bf16):
    x = workloads.activation(37, bpr, 3, 16 * bpr, outlier_frac=0.01, outlier_gain=30.0)
    _check(x, "per_row", bf16=bf16, what=f"per_row 3 x {16 * bpr} {'bf16' if bf16 else 'fp32'}")


def test_decode_weights_full():
    _check(workloads.DECODE.w(), what="decode w 5120x17408")


def test_fused_inputs_full():
    f = workloads.FUSED
    _check(f.x(), what="fused x 8192x5120")
    for i in range(len(f.widths)):
        _check(f.w(i), what=f"fused w{i}")


def test_sweep_down_projection_sampled_rows():
    # The largest activation of the sweep (16384 x 17408): GPU codes of sampled rows against
    # the oracle, whose per-tensor scale is the tensor's amax / 2688.
    sw = workloads.SWEEP
    x = sw.x(3, sw.mlp)
    xg = to_gpu(x)
    got = to_host(nv().quantize(xg))
    sg = ref.global_scale(x, ref.PER_TENSOR)
    assert got.global_scale.view(np.uint32)[0] == sg.view(np.uint32)[0]
    rows = np.random.default_rng(0).choice(sw.M, 64, replace=False)
    want = ref.quantize(x[rows], ref.GIVEN, float(sg[0]))
    assert_quant_equal(got, want, rows=rows, what="sweep mlp_down x")


@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (37, 80), (257, 256), (5, 4096 + 16)])
@pytest.mark.parametrize("mode", ["per_tensor", "per_row"])
def test_ragged_shapes(rows, cols, mode):
    x = workloads.activation(21, rows, rows, cols, outlier_frac=0.05)
    _check(x, mode, what=f"{rows}x{cols} {mode}")
    _check(x, mode, bf16=False, what=f"{rows}x{cols} {mode} fp32")


def test_row_pitch_larger_than_width():
    base = workloads.activation(22, 0, 40, 512)
    xg = to_gpu(base)[:, :384]              # row stride 512, width 384
    got = nv().quantize(xg)
    want = ref.quantize(xg.float().cpu().numpy())
    assert_quant_equal(got, want, what="strided")


@pytest.mark.parametrize("sg", [1.0, 0.37, 2.0 ** -7, 3.0e-5, 2.0 ** 20])
def test_every_code_with_every_scale(sg):
    sg = np.float32(sg)
    s_bytes = np.arange(1, 0x7F)
    d = (ref.e4m3_decode(s_bytes).astype(np.float32) * sg).astype(np.float32)
    x = (ref.e2m1_decode(np.arange(16)).astype(np.float32)[None, :] * d[:, None]).astype(np.float32)
    got, _ = _check(x.reshape(1, -1), "given", bf16=False, given=float(sg), what=f"exhaustive sg={sg}")
    h = to_host(got)
    assert np.array_equal(h.scales[0], s_bytes.astype(np.uint8))
    assert np.array_equal(ref.unpack_codes(h.codes).reshape(-1, 16), np.tile(np.arange(16), (126, 1)))


def test_ties_and_signed_zero():
    x = np.array([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                   -0.0]], np.float32)
    _check(x, "given", bf16=False, given=1.0, what="ties")
    _check(x * np.float32(2.0 ** -100), "given", bf16=False, given=2.0 ** -100, what="ties tiny scale")


def test_all_zero_and_empty():
    _check(np.zeros((7, 64), np.float32), what="zero tensor")
    _check(np.zeros((7, 64), np.float32), "per_row", what="zero rows")
    got = nv().quantize(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV))
    assert got.global_scale.item() == 0.0 and got.codes.numel() == 0


def test_subnormal_and_extreme_ranges():
    x = workloads.activation(23, 0, 16, 256, outlier_frac=0.02, bf16=False)
    for scale in (1e-38, 1e-30, 3e-41, 1e30, 1e35):
        _check((x * np.float32(scale)).astype(np.float32), bf16=False, what=f"scale {scale}")
        _check((x * np.float32(scale)).astype(np.float32), "per_row", bf16=False, what=f"row scale {scale}")
    # given scales far from the data: tiny d (slow division path) and saturated block scales
    for sg in (1e-40, 1e-30, 1e-3, 1e3):
        _check(x, "given", bf16=False, given=sg, what=f"given {sg}")


def test_nonfinite_input_gives_nonfinite_global_scale():
    x = workloads.activation(24, 0, 6, 64)
    x[2, 9] = np.nan
    got = nv().quantize(to_gpu(x))
    assert np.isnan(got.global_scale.item())
    gr = nv().quantize(to_gpu(x), "per_row").global_scale.cpu().numpy()
    assert np.isnan(gr[2]) and np.isfinite(np.delete(gr, 2)).all()
    x[2, 9] = -np.inf
    assert np.isinf(nv().quantize(to_gpu(x)).global_scale.item())


def test_deterministic():
    x = to_gpu(workloads.PREFILL.x(512))
    a, b = nv().quantize(x), nv().quantize(x)
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert torch.equal(a.global_scale, b.global_scale)


@pytest.mark.parametrize("sg", [1.0, 2.0 ** -10, 3.7, 2.0 ** 20])
@pytest.mark.parametrize("arrangement", ["sorted", "shuffled"])
def test_every_finite_bf16_value(sg, arrangement):
    # All 65280 finite bf16 bit patterns (both signs, subnormals and zeros included), in blocks of
    # 16 neighbouring magnitudes or randomly mixed, encoded under a given global scale.
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    if arrangement == "sorted":
        vals = vals[np.argsort(np.abs(vals), kind="stable")]
    else:
        vals = vals[np.random.default_rng(7).permutation(vals.size)]
    x = vals.reshape(-1, 256)                # 255 rows x 256 columns, exact in bf16
    assert x.shape[0] * 256 == vals.size
    _check(x, "given", bf16=True, given=sg, what=f"all bf16 {arrangement} sg={sg}")


@pytest.mark.parametrize("sg", [1.0, 2.0 ** -40, 2.0 ** 40])
def test_random_fp32_blocks_across_the_range(sg):
    # fp32 inputs with full random mantissas; each 16-block spans 4 octaves around its own
    # exponent in [-100, 100], so the quotient takes the fast and the fallback path alike.
    g = np.random.default_rng(11)
    nblk = 1 << 17
    e_blk = g.integers(-100, 101, nblk)
    e = np.repeat(e_blk, 16) - g.integers(0, 5, nblk * 16)
    m = 1.0 + g.random(nblk * 16)
    sgn = np.where(g.random(nblk * 16) < 0.5, -1.0, 1.0)
    x = (sgn * np.ldexp(m, e)).astype(np.float32).reshape(-1, 1024)
    assert np.isfinite(x).all()
    _check(x, "given", bf16=False, given=sg, what=f"random fp32 sg={sg}")
