"""CPU check that the every-scale-byte GEMM cases are sensitive to the decoding of each byte:
an oracle that flushed the subnormal E4M3 scales (bytes 0x01 to 0x07) to zero, or that read
one byte's exponent wrongly, produces outputs that the GPU tests' tolerance rejects.  The
mistake is planted in a copy of the oracle's decoding, never in GPU code."""
import numpy as np

from oracle import nvfp4_ref as ref
from tests.gpu_helpers import gemm_errors
from tests.test_gpu_scale_bytes import NBYTES, _a_operand, _operand


def _gemm_with(decode, oa, ow):
    saved = ref.e4m3_decode
    ref.e4m3_decode = decode
    try:
        return ref.gemm(oa, ow)[0]
    finally:
        ref.e4m3_decode = saved


def _rows_failing(oa, ow, Y_bad):
    """Rows of A whose outputs a correct kernel-like result (the oracle's own) and the
    planted-mistake result separate beyond the fp32 tolerance."""
    import torch
    Y, T = ref.gemm(oa, ow)
    err, bound = gemm_errors(torch.from_numpy(Y_bad.astype(np.float32)), Y, T)
    return np.unique(np.argwhere(~(err <= bound))[:, 0])


def test_flushed_subnormal_scales_are_caught():
    K = 256
    oa = _a_operand(11, 127, K, 0, True)
    ow = _operand(12, 300, K, 5, [0.75])
    good = ref.e4m3_decode

    def flushed(b):
        v = good(b)
        b = np.asarray(b)
        return np.where((b & 0x78) == 0, 0.0, v)

    bad_rows = _rows_failing(oa, ow, _gemm_with(flushed, oa, ow))
    # every A row whose byte is subnormal (1..7) fails, whatever the W byte
    assert set(range(1, 8)) <= set(bad_rows.tolist())


def test_one_wrong_byte_is_caught():
    K = 256
    oa = _a_operand(11, NBYTES, K, 0, False)
    ow = _operand(12, 300, K, 5, [0.75])
    good = ref.e4m3_decode
    for wrong in (0x01, 0x08, 0x3F, 0x7E):
        def off_by_one_exponent(b, wrong=wrong):
            b = np.asarray(b)
            return np.where(b == wrong, 2.0 * good(b), good(b))
        bad_rows = _rows_failing(oa, ow, _gemm_with(off_by_one_exponent, oa, ow))
        assert wrong in bad_rows.tolist()
