"""GPU parity of the GEMM over seeded random shapes that reach every kernel the launcher can
pick: the batch-1 matrix-vector kernel (M = 1, K % 64 == 0), the plain kernel (K % 128 != 0,
or more than 16 tokens with K % 256 != 0), the register decode kernel (M <= 16, K % 256 != 0),
the K-split and balanced decode kernels (M <= 16, K % 256 == 0, N on either side of one round of
32-row workgroups; the K-split kernel on 4 x 4 x 4 MFMAs for up to 4 tokens and N <= 20 x CUs) and
the prefill tiles with their peeled 128 x 128 tails.  Each case is a
fused launch of 1-4 modules with their own global scales (one module: the plain GEMM), per-
tensor or per-row activation scales and fp32 or bf16 output, checked element by element against
the oracle's fused GEMM with the per-element bound of the other parity tests.  The other entry
points (quantizer, one-call batch-1 decode, NVFP4-output, SwiGLU and GDN-gate epilogues, the
MXFP4 variant) get their own random sweeps, checked as their fixed-shape tests check them."""
import numpy as np
import pytest
import torch

import workloads
from oracle import nvfp4_ref as ref
from tests.gpu_helpers import assert_gemm_close, assert_quant_equal, nv, to_gpu

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(2024)
    cases = []
    # (M range, N range, K choices) per dispatch class
    classes = [
        ("batch-1", (1, 1), (1, 700), [64, 192, 320, 576, 2112, 4160]),
        ("plain K", (1, 40), (1, 200), [16, 48, 80, 144, 208, 400]),
        ("plain M>16", (17, 70), (1, 200), [128, 384, 640]),
        ("register decode", (2, 16), (1, 300), [128, 384, 896]),
        ("K-split decode", (2, 16), (1, 900), [256, 512, 1280, 2304]),
        ("balanced decode", (1, 16), (8193, 9400), [256, 512]),
        ("prefill tiles", (17, 300), (1, 700), [256, 512, 768]),
        # up to 4 tokens and N <= 20 x CUs: the K-split kernel on 4 x 4 x 4 MFMAs
        ("small-batch decode", (2, 4), (1, 5120), [256, 512, 1280, 2304]),
        # 5 to 8 tokens: the 16 x 16 x 32 K-split kernel copying one token chunk
        ("mid-batch decode", (5, 8), (1, 8192), [256, 512, 1280]),
    ]
    for name, (m0, m1), (n0, n1), ks in classes:
        for _ in range(10):
            M = int(rng.integers(m0, m1 + 1))
            N = int(rng.integers(n0, n1 + 1))
            K = int(rng.choice(ks))
            nseg = int(rng.integers(1, 5)) if N >= 4 else 1
            cuts = sorted(rng.choice(np.arange(1, N), size=nseg - 1, replace=False).tolist()) if nseg > 1 else []
            widths = [b - a for a, b in zip([0] + cuts, cuts + [N])]
            mode = "per_row" if rng.random() < 0.5 else "per_tensor"
            out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
            seed = int(rng.integers(0, 1 << 30))
            cases.append(pytest.param(M, K, tuple(widths), mode, out, seed, id=f"{name}-{M}x{N}x{K}-{len(widths)}seg"))
    return cases


@pytest.mark.parametrize("M,K,widths,mode,out_dtype,seed", _cases())
def test_random_shape(M, K, widths, mode, out_dtype, seed):
    xg = to_gpu(workloads.activation(seed, 0, M, K))
    a = nv().quantize(xg, mode)
    oa = ref.quantize(xg.float().cpu().numpy(), ref.PER_ROW if mode == "per_row" else ref.PER_TENSOR)
    assert_quant_equal(a, oa, what="A")
    gq, oq = [], []
    for i, n in enumerate(widths):
        wg = to_gpu(workloads.weight(seed, 1 + i, n, K, sigma=0.02 * (1 + i)))
        gq.append(nv().quantize(wg))
        oq.append(ref.quantize(wg.float().cpu().numpy()))
        assert_quant_equal(gq[-1], oq[-1], what=f"W{i}")
    # Half the cases write Y into a wider buffer (row pitch N + 8j elements, so both aligned and
    # unaligned rows) whose other columns must keep their sentinel.
    N = sum(widths)
    pitch = N if seed % 2 else N + 8 * (1 + seed % 7)
    big = torch.full((M, pitch), 7.0, dtype=out_dtype, device=xg.device)
    out = big[:, :N]
    if len(widths) == 1:
        y = nv().gemm(a, gq[0], out_dtype, out=out)
    else:
        y = nv().gemm_fused_segments(a, torch.cat([q.codes for q in gq]), torch.cat([q.scales for q in gq]),
                                     widths, torch.cat([q.global_scale for q in gq]), out_dtype, out=out)
    Y, T = ref.fused_segments(oa, oq)
    assert_gemm_close(y, Y, T, f"M={M} K={K} widths={widths} {mode} pitch {pitch}")
    assert bool((big[:, N:] == 7.0).all()), "columns past N were written"


def _quant_cases():
    rng = np.random.default_rng(7)
    cases = []
    for i in range(40):
        rows = int(rng.choice([0, 1, 2, 3, 17, 255, 256, 257, 1000, int(rng.integers(1, 3000))]))
        cols = 16 * int(rng.integers(1, 400))
        pad = 0 if rng.random() < 0.5 else 8 * int(rng.integers(1, 40))      # row stride - width, elements
        fp32 = bool(rng.random() < 0.3)
        mode = str(rng.choice(["per_tensor", "per_row", "given"]))
        cases.append(pytest.param(rows, cols, pad, fp32, mode, i, id=f"{rows}x{cols}+{pad}-{'f32' if fp32 else 'bf16'}-{mode}"))
    return cases


@pytest.mark.parametrize("rows,cols,pad,fp32,mode,seed", _quant_cases())
def test_random_quantize(rows, cols, pad, fp32, mode, seed):
    """Quantizer bytes (codes, scale bytes, global scales) bitwise against the oracle over random
    shapes, row strides wider than the rows, both input types and every scale mode."""
    # (the stride cols + pad is a multiple of 8 elements: 16-byte rows for both input types)
    x = workloads.activation(1000 + seed, 0, max(rows, 1), cols + pad)[:rows] * np.float32(1 + seed % 5)
    full = to_gpu(x, bf16=not fp32)
    xg = full[:, :cols]
    src = xg.float().cpu().numpy()
    # Outputs are the fronts of larger buffers holding a sentinel, which must survive.
    guard = 64
    cbuf = torch.full((rows * cols // 2 + guard,), 0xA5, dtype=torch.uint8, device=xg.device)
    sbuf = torch.full((rows * cols // 16 + guard,), 0x5A, dtype=torch.uint8, device=xg.device)
    ng = rows if mode == "per_row" else 1
    gbuf = torch.full((ng + guard,), -3.0, dtype=torch.float32, device=xg.device)
    out = nv().NVFP4Tensor(cbuf[:rows * cols // 2].view(rows, cols // 2), sbuf[:rows * cols // 16].view(rows, cols // 16),
                           gbuf[:ng])
    if mode == "given":
        g = torch.tensor([np.float32(0.0123 * (1 + seed % 7))], dtype=torch.float32, device=xg.device)
        gbuf[0] = g[0]
        got = nv().quantize(xg, "given", global_scale=gbuf[:1], out=out)
        want = ref.quantize(src, ref.GIVEN, given=float(g.item()))
    else:
        got = nv().quantize(xg, mode, out=out)
        want = ref.quantize(src, ref.PER_ROW if mode == "per_row" else ref.PER_TENSOR)
    assert_quant_equal(got, want, what=f"{rows}x{cols} stride {cols + pad}")
    assert bool((cbuf[rows * cols // 2:] == 0xA5).all()) and bool((sbuf[rows * cols // 16:] == 0x5A).all()), \
        "bytes past the codes or scale bytes were written"
    assert bool((gbuf[ng:] == -3.0).all()), "floats past the global scales were written"


def _decode_linear_cases():
    rng = np.random.default_rng(11)
    cases = []
    for i in range(24):
        K = 64 * int(rng.integers(1, 288))                   # up to the one-call kernel's LDS limit
        N = int(rng.choice([1, 3, int(rng.integers(1, 9000)), int(rng.integers(1, 300))]))
        mode = "per_tensor" if rng.random() < 0.7 else "given"
        cases.append(pytest.param(N, K, mode, i, id=f"{N}x{K}-{mode}"))
    return cases


@pytest.mark.parametrize("N,K,mode,seed", _decode_linear_cases())
def test_random_decode_linear(N, K, mode, seed):
    """The one-call batch-1 decode over random shapes: the token's bytes bitwise against the
    oracle's quantization of the bf16 row, Y against the oracle's product within the bound."""
    xg = to_gpu(workloads.activation(2000 + seed, 0, 1, K))
    wg = to_gpu(workloads.weight(2000 + seed, 1, N, K, sigma=0.03))
    w = nv().quantize(wg)
    ow = ref.quantize(wg.float().cpu().numpy())
    src = xg.float().cpu().numpy()
    # Y and the token's bytes go to the fronts of larger buffers holding a sentinel.
    dev, guard = xg.device, 64
    ybuf = torch.full((N + guard,), -7.0, dtype=torch.float32, device=dev)
    cbuf = torch.full((K // 2 + guard,), 0xA5, dtype=torch.uint8, device=dev)
    sbuf = torch.full((K // 16 + guard,), 0x5A, dtype=torch.uint8, device=dev)
    gbuf = torch.full((1 + guard,), -3.0, dtype=torch.float32, device=dev)
    a_out = nv().NVFP4Tensor(cbuf[:K // 2].view(1, K // 2), sbuf[:K // 16].view(1, K // 16), gbuf[:1])
    if mode == "given":
        gs = np.float32(0.004 * (1 + seed % 3))
        gbuf[0] = float(gs)
        y, a = nv().decode_linear(xg, w, mode="given", global_scale=gbuf[:1], out_dtype=torch.float32,
                                  out=ybuf[:N].view(1, N), a_out=a_out)
        oa = ref.quantize(src, ref.GIVEN, given=float(gs))
    else:
        y, a = nv().decode_linear(xg, w, mode="per_tensor", out_dtype=torch.float32, out=ybuf[:N].view(1, N),
                                  a_out=a_out)
        oa = ref.quantize(src, ref.PER_ROW)
    assert_quant_equal(a, oa, what="token")
    Y, T = ref.gemm(oa, ow)
    assert_gemm_close(y, Y, T, f"decode_linear N={N} K={K}")
    assert bool((ybuf[N:] == -7.0).all()), "floats past Y were written"
    assert bool((cbuf[K // 2:] == 0xA5).all()) and bool((sbuf[K // 16:] == 0x5A).all()), "token bytes overran"
    assert bool((gbuf[1:] == -3.0).all()), "floats past the token's global scale were written"


def _epilogue_shape(rng):
    """M, K for the fused epilogues: up to 16 tokens K a multiple of 128 (K-split or balanced
    decode kernel at K % 256 == 0, the register decode kernel otherwise), past 16 a multiple of
    256 (prefill tiles)."""
    M = int(rng.choice([1, int(rng.integers(2, 17)), int(rng.integers(17, 400))]))
    K = 128 * int(rng.integers(1, 24)) if M <= 16 else 256 * int(rng.integers(1, 12))
    return M, K


def _nvfp4_out_cases():
    rng = np.random.default_rng(17)
    cases = []
    for i in range(16):
        M, K = _epilogue_shape(rng)
        nseg = int(rng.integers(1, 4))
        widths = tuple(16 * int(rng.integers(1, 160)) for _ in range(nseg))
        mode = "per_row" if rng.random() < 0.5 else "per_tensor"
        cases.append(pytest.param(M, K, widths, mode, 300 + i, id=f"{M}x{K}-{'-'.join(map(str, widths))}-{mode}"))
    return cases


@pytest.mark.parametrize("M,K,widths,a_mode,seed", _nvfp4_out_cases())
def test_random_nvfp4_out(M, K, widths, a_mode, seed):
    """GEMM with NVFP4 output over random shapes: the fp32 values within the GEMM bound, then the
    codes and scale bytes bitwise against the oracle's encoding of them."""
    from tests.test_gpu_nvfp4_out import _check
    _check(M, K, widths, a_mode, seed=seed)


def _swiglu_cases():
    rng = np.random.default_rng(19)
    cases = []
    for i in range(16):
        M, K = _epilogue_shape(rng)
        F = 16 * int(rng.integers(1, 300))
        h = torch.bfloat16 if rng.random() < 0.5 else torch.float32
        mode = ref.PER_ROW if rng.random() < 0.5 else ref.PER_TENSOR
        cases.append(pytest.param(M, F, K, mode, h, 400 + i, id=f"{M}x{F}x{K}-{mode}-{str(h)[6:]}"))
    return cases


@pytest.mark.parametrize("M,F,K,a_mode,h_dtype,seed", _swiglu_cases())
def test_random_swiglu(M, F, K, a_mode, h_dtype, seed):
    """The SwiGLU GEMM over random shapes: h within its derived bound, NVFP4 h bitwise."""
    from tests.test_gpu_swiglu import _check, _workload_operands
    oa, og, ou = _workload_operands(seed, M, F, K, a_mode)
    _check(oa, og, ou, h_dtype, what=f"swiglu {M}x{F}x{K}")


def _gdn_cases():
    rng = np.random.default_rng(23)
    cases = []
    for i in range(12):
        M, K = _epilogue_shape(rng)
        H = int(rng.integers(1, 65))
        lead = tuple(int(rng.integers(1, 600)) for _ in range(int(rng.integers(1, 4))))
        mode = "per_row" if rng.random() < 0.5 else "per_tensor"
        out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
        cases.append(pytest.param(M, K, lead + (H, H), mode, out, 500 + i,
                                  id=f"{M}x{K}-{'-'.join(map(str, lead))}-H{H}-{mode}"))
    return cases


@pytest.mark.parametrize("M,K,widths,a_mode,out_dtype,seed", _gdn_cases())
def test_random_gdn_gates(M, K, widths, a_mode, out_dtype, seed):
    """The fused GDN projection with its gate epilogue over random shapes and head counts: Y
    within the GEMM bound and bitwise equal to the fused GEMM, the gates within their bound."""
    from tests.test_gpu_gdn_gates import _run
    _run(M, K, widths, seed, a_mode, out_dtype=out_dtype)


def _mx_cases():
    rng = np.random.default_rng(29)
    cases = []
    for i in range(12):
        M = int(rng.choice([1, int(rng.integers(2, 17)), int(rng.integers(17, 400))]))
        N = int(rng.integers(1, 1200))
        K = 256 * int(rng.integers(1, 12))
        out = torch.bfloat16 if rng.random() < 0.5 else torch.float32
        cases.append(pytest.param(M, N, K, out, 600 + i, id=f"{M}x{N}x{K}-{str(out)[6:]}"))
    return cases


@pytest.mark.parametrize("M,N,K,out_dtype,seed", _mx_cases())
def test_random_mxfp4(M, N, K, out_dtype, seed):
    """The lossy MXFP4 variant over random shapes: re-encoding bitwise against the oracle, the
    GEMM within the bound against the oracle's product of the re-encoded operands."""
    from tests.test_gpu_mxfp4 import _mx_pair
    ma, mw, oma, omw, _, _ = _mx_pair(M, N, K, seed)
    y = nv().mxfp4_gemm(ma, mw.codes, mw.scales, (N,), mw.global_scale, out_dtype)
    Y, T = ref.mx_gemm(oma, omw)
    assert_gemm_close(y, Y, T, f"mx {M}x{N}x{K}")


def _guarded(shape, dtype, fill, dev, guard=64):
    """A tensor of `shape` at the front of a buffer whose `guard` trailing elements hold `fill`."""
    n = int(np.prod(shape))
    buf = torch.full((n + guard,), fill, dtype=dtype, device=dev)
    return buf, buf[:n].view(*shape)


def _tail_intact(buf, n, fill):
    return bool((buf[n:] == fill).all())


def _bounds_cases():
    rng = np.random.default_rng(31)
    cases = []
    for i in range(12):
        M, K = _epilogue_shape(rng)
        widths = tuple(16 * int(rng.integers(1, 120)) for _ in range(int(rng.integers(1, 4))))
        cases.append(pytest.param(M, K, widths, 700 + i, id=f"{M}x{K}-{'-'.join(map(str, widths))}"))
    return cases


@pytest.mark.parametrize("M,K,widths,seed", _bounds_cases())
def test_random_epilogue_writes_stay_in_bounds(M, K, widths, seed):
    """The NVFP4-output, SwiGLU and GDN-gate epilogues write their outputs into the fronts of
    larger buffers holding a sentinel: every element past each output must survive (the values
    are checked by the sweeps above)."""
    dev = torch.device("cuda:0")
    a = nv().quantize(to_gpu(workloads.activation(seed, 0, M, K)), "per_row" if seed % 2 else "per_tensor")
    qs = [nv().quantize(to_gpu(workloads.weight(seed, 1 + i, n, K))) for i, n in enumerate(widths)]
    wc, ws = torch.cat([q.codes for q in qs]), torch.cat([q.scales for q in qs])
    wg = torch.cat([q.global_scale for q in qs])
    N = sum(widths)
    # NVFP4 output
    cb, c = _guarded((M, N // 2), torch.uint8, 0xA5, dev)
    sb, s = _guarded((M, N // 16), torch.uint8, 0x5A, dev)
    yg = torch.tensor([0.01], dtype=torch.float32, device=dev)
    nv().gemm_nvfp4_out(a, wc, ws, widths, wg, yg, out=nv().NVFP4Tensor(c, s, yg))
    assert _tail_intact(cb, M * N // 2, 0xA5) and _tail_intact(sb, M * N // 16, 0x5A), "NVFP4 output overran"
    # SwiGLU on the first module as gate and up (F = its width)
    F = widths[0]
    gcodes, gscales = nv().interleave_gate_up(qs[0], qs[0])
    hb, h = _guarded((M, F), torch.float32, -7.0, dev)
    hcb, hc = _guarded((M, F // 2), torch.uint8, 0xA5, dev)
    hsb, hs = _guarded((M, F // 16), torch.uint8, 0x5A, dev)
    nv().gemm_swiglu(a, gcodes, gscales, torch.cat([qs[0].global_scale, qs[0].global_scale]),
                     h_dtype=torch.float32, h_global=yg, out=h, q_out=nv().NVFP4Tensor(hc, hs, yg))
    assert _tail_intact(hb, M * F, -7.0), "SwiGLU h overran"
    assert _tail_intact(hcb, M * F // 2, 0xA5) and _tail_intact(hsb, M * F // 16, 0x5A), "NVFP4 h overran"
    # GDN gates on the modules plus two gate segments of H heads
    H = 1 + seed % 40
    gq = [nv().quantize(to_gpu(workloads.weight(seed, 10 + j, H, K, sigma=0.05))) for j in range(2)]
    gw = tuple(widths) + (H, H)
    gc2 = torch.cat([wc] + [q.codes for q in gq])
    gs2 = torch.cat([ws] + [q.scales for q in gq])
    gg2 = torch.cat([wg] + [q.global_scale for q in gq])
    a_log = torch.linspace(-1.0, 1.0, H, device=dev)
    dt = torch.linspace(-0.5, 0.5, H, device=dev)
    yb, y = _guarded((M, N + 2 * H), torch.float32, -7.0, dev)
    gb, g = _guarded((M, H), torch.float32, -7.0, dev)
    bb, beta = _guarded((M, H), torch.float32, -7.0, dev)
    nv().gemm_fused_gdn_gates(a, gc2, gs2, gw, gg2, a_log, dt, torch.float32, out=y, g_out=g, beta_out=beta)
    assert _tail_intact(yb, M * (N + 2 * H), -7.0), "fused output overran"
    assert _tail_intact(gb, M * H, -7.0) and _tail_intact(bb, M * H, -7.0), "gate outputs overran"
