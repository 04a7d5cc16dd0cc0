"""GPU parity of the batch-1 decode entry point (nvfp4_decode_linear): quantize one token and
multiply it with W in one call.  Its contract is the two-call sequence quantize -> gemm on the
same inputs: the token's NVFP4 bytes and global scale bit for bit, and Y bit for bit wherever the
plain GEMM takes the batch-1 matrix-vector kernel as well (N up to one round of 32-row
workgroups, or K not a multiple of 256); elsewhere (the up projection) Y is checked against the
oracle's GEMM of the same bytes within the GEMM bound.  bf16 tokens with K a multiple of 64 whose
working set fits the kernel's LDS (K up to 18432 here) run the fused kernel; fp32 tokens and other
K run the two calls inside the library."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import DEV, assert_gemm_close, assert_quant_equal, nv, to_gpu, to_host

pytestmark = pytest.mark.gpu


def _bitwise(x: torch.Tensor, N: int, K: int) -> bool:
    """False only where the fused kernel may run while the plain GEMM takes an MFMA kernel."""
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    return not (x.dtype == torch.bfloat16 and K % 256 == 0 and N > 32 * cus)


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


def _weight(N: int, K: int, seed: int):
    w = to_gpu(workloads.weight(seed, 1, N, K))
    q = nv().quantize(w)
    return q, w


def _check(x: torch.Tensor, q, mode: str, out_dtype, what: str, given=None, oracle=None):
    a2 = nv().quantize(x, mode, given)
    y2 = nv().gemm(a2, q, out_dtype)
    y1, a1 = nv().decode_linear(x, q, mode, given, out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(a1.codes, a2.codes), f"{what}: token codes"
    assert torch.equal(a1.scales, a2.scales), f"{what}: token scale bytes"
    assert np.array_equal(_bits(a1.global_scale), _bits(a2.global_scale)), f"{what}: global scale"
    N, K = q.rows, q.cols
    if _bitwise(x, N, K):
        assert np.array_equal(_bits(y1), _bits(y2)), f"{what}: Y differs from quantize + gemm"
    if oracle is not None:
        Y, T = ref.gemm(to_host(a1), oracle)
        assert_gemm_close(y1, Y, T, what)
    return y1, a1


@pytest.mark.parametrize("N,K", [(5120, 17408), (1, 64), (7, 320), (300, 4160), (2048, 18432), (600, 32768),
                                 (64, 32832), (100, 1040), (17408, 5120)])
def test_decode_linear_matches_quantize_then_gemm(N, K):
    # Shapes: the MLP down projection; one 32-value group; short rows over many wavefronts; the
    # longest row the fused kernel's LDS holds (K = 18432) and rows it does not (K = 32768 and
    # 32832: two calls); K not a multiple of 64 (two calls); the up projection (fused kernel; the
    # plain GEMM takes the balanced MFMA kernel there, so Y is checked against the oracle).
    q, w = _weight(N, K, 40 + K % 97)
    ow = ref.quantize(w.float().cpu().numpy())
    assert_quant_equal(q, ow, what="W")
    x = to_gpu(workloads.activation(41, N % 89, 1, K, outlier_frac=0.01))
    for mode in ("per_tensor", "per_row"):
        for dt in (torch.bfloat16, torch.float32):
            _check(x, q, mode, dt, f"1x{N}x{K} {mode} {dt}", oracle=ow if mode == "per_tensor" else None)
    # the token itself against the oracle's quantizer
    _, a1 = nv().decode_linear(x, q)
    assert_quant_equal(a1, ref.quantize(x.float().cpu().numpy(), ref.PER_ROW), what="token")


def test_decode_linear_given_scale_and_fp32_token():
    N, K = 5120, 17408
    q, w = _weight(N, K, 42)
    ow = ref.quantize(w.float().cpu().numpy())
    xb = to_gpu(workloads.activation(43, 0, 1, K))
    given = torch.tensor([float(np.float32(3.5 / 2688))], dtype=torch.float32, device=DEV)
    y, a = _check(xb, q, "given", torch.float32, "given scale", given=given, oracle=ow)
    assert a.global_scale.data_ptr() == given.data_ptr()
    # an fp32 token takes the two calls inside the library: the same contract
    xf = to_gpu(workloads.activation(43, 1, 1, K), bf16=False)
    _check(xf, q, "per_tensor", torch.bfloat16, "fp32 token", oracle=ow)


@pytest.mark.parametrize("case", ["zeros", "nan", "inf", "huge", "tiny", "one_outlier"])
def test_decode_linear_special_tokens(case):
    # Special rows through the fused quantization: the bytes and Y must still be those of the two
    # calls (all-zero row: global scale 0; NaN and inf propagate through the row maximum).
    N, K = 300, 4160
    q, _ = _weight(N, K, 44)
    x = workloads.activation(45, 0, 1, K)
    if case == "zeros":
        x[:] = 0.0
    elif case == "nan":
        x[0, 1000] = np.nan
    elif case == "inf":
        x[0, 7] = -np.inf
    elif case == "huge":
        x *= np.float32(3e36)
    elif case == "tiny":
        x *= np.float32(1e-36)
    else:
        x[0, 4000] = 1e4
    _check(to_gpu(x), q, "per_tensor", torch.float32, case)


def test_decode_linear_quantize_only():
    # N = 0: only the token's quantization.
    K = 640
    x = to_gpu(workloads.activation(46, 0, 1, K))
    w = nv().NVFP4Tensor(torch.empty((0, K // 2), dtype=torch.uint8, device=DEV),
                         torch.empty((0, K // 16), dtype=torch.uint8, device=DEV),
                         torch.ones(1, dtype=torch.float32, device=DEV))
    y, a = nv().decode_linear(x, w)
    assert y.shape == (1, 0)
    assert_quant_equal(a, ref.quantize(x.float().cpu().numpy(), ref.PER_ROW), what="token")


def test_decode_linear_repeated_calls_deterministic():
    N, K = 5120, 17408
    q, _ = _weight(N, K, 47)
    x = to_gpu(workloads.activation(48, 0, 1, K))
    y0, _ = nv().decode_linear(x, q, out_dtype=torch.float32)
    for _ in range(5):
        y, _ = nv().decode_linear(x, q, out_dtype=torch.float32)
        assert torch.equal(y, y0)
