"""CPU checks of the Python binding's argument checks: every malformed tensor argument raises
ValueError before the library is called.  The binding checks shapes, dtypes, contiguity and
global-scale counts first and GPU residency last, so these cases run on CPU tensors; a call
whose only fault is that its tensors live on the CPU fails the residency check."""
import numpy as np
import pytest
import torch


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_block_amd as m
    return m


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def f32(*shape):
    return torch.ones(shape, dtype=torch.float32)


def operand(nv, R, K, gs=1, group=16):
    return nv.NVFP4Tensor(u8(R, K // 2), u8(R, K // group), f32(gs))


def test_quantize_out_checked(nv):
    x = torch.zeros((8, 64), dtype=torch.bfloat16)
    bad_codes = nv.NVFP4Tensor(u8(8, 16), u8(8, 4), f32(1))
    with pytest.raises(ValueError, match="out.codes"):
        nv.quantize(x, out=bad_codes)
    bad_scales = nv.NVFP4Tensor(u8(8, 32), u8(8, 2), f32(1))
    with pytest.raises(ValueError, match="out.scales"):
        nv.quantize(x, out=bad_scales)
    # per-row mode writes one scale per row: a one-element buffer is refused
    with pytest.raises(ValueError, match="global scale"):
        nv.quantize(x, "per_row", out=nv.NVFP4Tensor(u8(8, 32), u8(8, 4), f32(1)))
    with pytest.raises(ValueError, match="global scale"):
        nv.quantize(x, out=nv.NVFP4Tensor(u8(8, 32), u8(8, 4), torch.ones(1, dtype=torch.float64)))
    with pytest.raises(ValueError, match="contiguous"):
        nv.quantize(x, out=nv.NVFP4Tensor(u8(8, 64)[:, :32], u8(8, 4), f32(1)))
    with pytest.raises(ValueError, match="mode"):
        nv.quantize(x, "per_column")
    with pytest.raises(ValueError, match="GPU"):          # well-formed, but on the CPU
        nv.quantize(x)
    with pytest.raises(ValueError, match="row-contiguous"):
        nv.quantize(torch.zeros((8, 128), dtype=torch.bfloat16)[:, ::2])
    # no rows: no data, so any strides pass the layout checks (torch gives (0, 0) for an empty
    # array made from numpy); only the residency check remains
    with pytest.raises(ValueError, match="GPU"):
        nv.quantize(torch.from_numpy(np.zeros((0, 64), np.float32)))


def test_gemm_operands_checked(nv):
    a, w = operand(nv, 4, 64), operand(nv, 8, 64)
    with pytest.raises(ValueError, match="GPU"):
        nv.gemm(a, w)
    # a column slice of the codes would be read at pitch K/2
    sliced = nv.NVFP4Tensor(u8(4, 64)[:, :32], u8(4, 4), f32(1))
    with pytest.raises(ValueError, match="contiguous"):
        nv.gemm(sliced, w)
    with pytest.raises(ValueError, match="scales"):
        nv.gemm(nv.NVFP4Tensor(u8(4, 32), u8(4, 3), f32(1)), w)
    with pytest.raises(ValueError, match="w.global_scale"):
        nv.gemm(a, operand(nv, 8, 64, gs=8))
    # the activation's global scales: one, or one per row; a row slice of a per-row tensor
    # that keeps all the scales is refused rather than read as per-tensor
    with pytest.raises(ValueError, match="a.global_scale"):
        nv.gemm(operand(nv, 4, 64, gs=16), w)
    with pytest.raises(ValueError, match="K mismatch"):
        nv.gemm(a, operand(nv, 8, 128))
    with pytest.raises(ValueError, match="out"):
        nv.gemm(a, w, torch.float32, out=f32(4, 9))


def test_fused_weights_checked(nv):
    a = operand(nv, 4, 64)
    wc, ws = u8(24, 32), u8(24, 4)
    with pytest.raises(ValueError, match="GPU"):
        nv.gemm_fused_segments(a, wc, ws, (16, 8), f32(2))
    with pytest.raises(ValueError, match="w_globals"):
        nv.gemm_fused_segments(a, wc, ws, (16, 8), f32(1))
    with pytest.raises(ValueError, match="w_codes"):
        nv.gemm_fused_segments(a, u8(20, 32), ws, (16, 8), f32(2))
    with pytest.raises(ValueError, match="w_scales"):
        nv.gemm_fused_segments(a, wc, u8(24, 8)[:, :4], (16, 8), f32(2))
    with pytest.raises(ValueError, match="positive"):
        nv.gemm_fused_segments(a, wc, ws, (24, 0), f32(2))
    with pytest.raises(ValueError, match="w_globals"):
        nv.gemm_nvfp4_out(a, wc, ws, (16, 8), f32(3), f32(1))
    with pytest.raises(ValueError, match="y_global"):
        nv.gemm_nvfp4_out(a, wc, ws, (16, 8), f32(2), f32(2))
    with pytest.raises(ValueError, match="out.codes"):
        nv.gemm_nvfp4_out(a, wc, ws, (16, 8), f32(2), f32(1), out=nv.NVFP4Tensor(u8(4, 8), u8(4, 1), f32(1)))


def test_gates_swiglu_mxfp4_checked(nv):
    a = operand(nv, 4, 64)
    wc, ws = u8(24, 32), u8(24, 4)
    with pytest.raises(ValueError, match="a_log"):
        nv.gemm_fused_gdn_gates(a, wc, ws, (8, 8, 8), f32(3), f32(4), f32(8))
    with pytest.raises(ValueError, match="gates"):
        nv.gemm_fused_gdn_gates(a, wc, ws, (8, 12, 4), f32(3), f32(4), f32(4))
    with pytest.raises(ValueError, match="GPU"):
        nv.gemm_fused_gdn_gates(a, wc, ws, (8, 8, 8), f32(3), f32(8), f32(8))
    with pytest.raises(ValueError, match="w_globals"):
        nv.gemm_swiglu(a, u8(32, 32), u8(32, 4), f32(1))
    with pytest.raises(ValueError, match="h_global"):
        nv.gemm_swiglu(a, u8(32, 32), u8(32, 4), f32(2), h_global=f32(2))
    with pytest.raises(ValueError, match="GPU"):
        nv.gemm_swiglu(a, u8(32, 32), u8(32, 4), f32(2))
    am = nv.MXFP4Tensor(u8(4, 32), u8(4, 2), f32(1))
    with pytest.raises(ValueError, match="w_scales"):
        nv.mxfp4_gemm(am, u8(8, 32), u8(8, 4), (8,), f32(1))
    with pytest.raises(ValueError, match="GPU"):
        nv.mxfp4_gemm(am, u8(8, 32), u8(8, 2), (8,), f32(1))
    with pytest.raises(ValueError, match="out.scales"):
        nv.to_mxfp4(operand(nv, 4, 64), out=nv.MXFP4Tensor(u8(4, 32), u8(4, 4), f32(1)))
    with pytest.raises(ValueError, match="same shape"):
        nv.interleave_gate_up(operand(nv, 16, 64), operand(nv, 32, 64))


def test_fp8_kv_checked(nv):
    x = torch.zeros(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="scale"):
        nv.fp8_kv_quantize(x, f32(2))
    with pytest.raises(ValueError, match="out"):
        nv.fp8_kv_quantize(x, f32(1), out=u8(32))
    with pytest.raises(ValueError, match="GPU"):
        nv.fp8_kv_quantize(x, f32(1))
    with pytest.raises(ValueError, match="GPU"):
        nv.fp8_kv_dequantize(u8(64), f32(1))


def test_decode_linear_checked(nv):
    x = torch.zeros((1, 64), dtype=torch.bfloat16)
    w = operand(nv, 8, 64)
    with pytest.raises(ValueError, match="GPU"):          # well-formed, but on the CPU
        nv.decode_linear(x, w)
    with pytest.raises(ValueError, match=r"\[1, K\]"):
        nv.decode_linear(torch.zeros((2, 64), dtype=torch.bfloat16), w)
    with pytest.raises(ValueError, match="bf16 or fp32"):
        nv.decode_linear(torch.zeros((1, 64), dtype=torch.float16), w)
    with pytest.raises(ValueError, match="K mismatch"):
        nv.decode_linear(x, operand(nv, 8, 128))
    with pytest.raises(ValueError, match="mode"):
        nv.decode_linear(x, w, "per_column")
    with pytest.raises(ValueError, match="global_scale"):
        nv.decode_linear(x, w, "given")
    with pytest.raises(ValueError, match="w.global_scale"):
        nv.decode_linear(x, operand(nv, 8, 64, gs=8))
    with pytest.raises(ValueError, match="a_out.codes"):
        nv.decode_linear(x, w, a_out=nv.NVFP4Tensor(u8(1, 16), u8(1, 4), f32(1)))
    with pytest.raises(ValueError, match="a_out.global_scale"):
        nv.decode_linear(x, w, a_out=nv.NVFP4Tensor(u8(1, 32), u8(1, 4), f32(2)))
