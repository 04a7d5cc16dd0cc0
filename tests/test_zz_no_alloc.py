"""GPU check of nvfp4_quantize_no_alloc, the quantize entry point that allocates nothing (its
per-tensor partial maxima live in a static device array of the library): called through the C
ABI, its codes, scale bytes and global scales equal those of nvfp4_quantize with a workspace,
bit for bit, on two calls in a row (the second smaller, so stale contents of the shared array
from the first call would show), in every scale mode, and per tensor on bf16 and fp32 shapes
from one block to 16384 x 5120."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import DEV, nv, to_gpu

pytestmark = pytest.mark.gpu


def _outs(rows, cols, mode, given=None):
    codes = torch.full((rows, cols // 2), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, cols // 16), 0xCD, dtype=torch.uint8, device=DEV)
    if mode == nv().GIVEN:
        g = given
    else:
        g = torch.full((rows if mode == nv().PER_ROW else 1,), -1.0, dtype=torch.float32, device=DEV)
    return codes, scales, g


def _no_alloc(x, mode, given=None):
    rows, cols = x.shape
    codes, scales, g = _outs(rows, cols, mode, given)
    st = nv().lib.nvfp4_quantize_no_alloc(x.data_ptr(), 1 if x.dtype == torch.bfloat16 else 0, rows, cols,
                                          x.stride(0), codes.data_ptr(), scales.data_ptr(), g.data_ptr(), mode,
                                          torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 0, nv().lib.nvfp4_status_string(st)
    return codes, scales, g


def _with_workspace(x, mode, given=None):
    rows, cols = x.shape
    codes, scales, g = _outs(rows, cols, mode, given)
    wsb = nv().lib.nvfp4_quantize_workspace_size(rows, cols, mode)
    ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=DEV)
    st = nv().lib.nvfp4_quantize(x.data_ptr(), 1 if x.dtype == torch.bfloat16 else 0, rows, cols, x.stride(0),
                                 codes.data_ptr(), scales.data_ptr(), g.data_ptr(), mode, ws.data_ptr(), wsb,
                                 torch.cuda.current_stream(DEV).cuda_stream)
    assert st == 0, nv().lib.nvfp4_status_string(st)
    return codes, scales, g


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_no_alloc_matches_workspace_entry(mode):
    given = torch.tensor([0.0125], dtype=torch.float32, device=DEV)
    # the prefill activation (4096 x 5120 bf16, 0.1 % x50 outlier channels), then a smaller one
    # with a different maximum: the second call must not see the first call's partial maxima
    shapes = [(4096, 5120, 1), (300, 1024, 2)]
    for rows, cols, seed in shapes:
        x = to_gpu(workloads.activation(seed, 7, rows, cols, outlier_frac=0.001, outlier_gain=50.0 / seed))
        got = _no_alloc(x, mode, given)
        want = _with_workspace(x, mode, given)
        torch.cuda.synchronize()
        for a, b, name in zip(got, want, ("codes", "scales", "global scale")):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), (rows, cols, mode, name)


# Per-tensor shapes from one 16-element block to the sweep's 16384 x 5120 activation, bf16 and fp32.
@pytest.mark.parametrize("rows,cols,bf16", [(4096, 5120, True), (8192, 5120, True), (16384, 5120, True),
                                            (1000, 4096, False), (5120, 4096, False), (3, 48, True),
                                            (1, 16, False)])
def test_no_alloc_per_tensor_shapes(rows, cols, bf16):
    x = to_gpu(workloads.activation(6, rows, rows, cols, outlier_frac=0.01), bf16)
    for _ in range(2):                       # the second call finds what the first left in the array
        got = _no_alloc(x, 0)
        want = _with_workspace(x, 0)
        torch.cuda.synchronize()
        for a, b, name in zip(got, want, ("codes", "scales", "global scale")):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rows, cols, bf16, name)


def test_no_alloc_second_call_smaller_max():
    # The first call's tensor has a far larger maximum than the second's: a stale partial max
    # left in the shared array would inflate the second call's global scale.
    big = torch.full((512, 2048), 1000.0, dtype=torch.bfloat16, device=DEV)
    small = to_gpu(workloads.activation(5, 8, 64, 256))
    _no_alloc(big, 0)
    _, _, g = _no_alloc(small, 0)
    want = np.float32(np.abs(small.float().cpu().numpy()).max()) / np.float32(2688.0)
    assert g.item() == float(want)


def test_no_alloc_argument_errors():
    f = nv().lib.nvfp4_quantize_no_alloc
    x = torch.zeros((4, 32), dtype=torch.bfloat16, device=DEV)
    c = torch.empty((4, 16), dtype=torch.uint8, device=DEV)
    s = torch.empty((4, 2), dtype=torch.uint8, device=DEV)
    g = torch.empty((1,), dtype=torch.float32, device=DEV)
    assert f(x.data_ptr(), 1, 4, 24, 32, c.data_ptr(), s.data_ptr(), g.data_ptr(), 0, None) == 1   # cols % 16
    assert f(None, 1, 4, 32, 32, c.data_ptr(), s.data_ptr(), g.data_ptr(), 0, None) == 1
    assert f(x.data_ptr(), 1, 4, 32, 32, c.data_ptr(), s.data_ptr(), g.data_ptr(), 9, None) == 1   # mode
