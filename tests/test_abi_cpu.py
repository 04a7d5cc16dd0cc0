"""CPU checks of the C-ABI library: it loads, exports every function the header declares,
and rejects bad arguments on the host before touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_block_amd as m
    return m


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    fns = _declared_functions()
    for f in ("nvfp4_quantize", "nvfp4_gemm", "nvfp4_gemm_fused_segments"):
        assert f in fns


def test_library_exports_every_declared_function(nv):
    out = subprocess.run(["nm", "-D", "--defined-only", nv.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (nvfp4_[a-z0-9_]+)", out))
    missing = [f for f in _declared_functions() if f not in exported]
    assert not missing, missing
    assert set(nv.EXPORTED_SYMBOLS) == set(_declared_functions())
    for f in _declared_functions():
        assert hasattr(ctypes.CDLL(nv.library_path()), f)


def test_status_strings(nv):
    for s in range(5):
        assert nv.lib.nvfp4_status_string(s)
    assert nv.lib.nvfp4_status_string(99) == b"unknown status"
    assert nv.lib.nvfp4_version() >= 100


# Host-side validation: every call below must return before any HIP call.  Pointers are
# fake addresses, never dereferenced.
A16 = 0x10000
MIS = 0x10001


def q(nv, x=A16, dt=1, rows=4, cols=32, ldx=32, codes=A16, scales=A16, g=A16, mode=2, ws=None, wsb=0):
    return nv.lib.nvfp4_quantize(x, dt, rows, cols, ldx, codes, scales, g, mode, ws, wsb, None)


def test_quantize_argument_errors(nv):
    assert q(nv, cols=24, ldx=24) == 1             # cols not a multiple of 16
    assert q(nv, cols=0, ldx=0) == 1
    assert q(nv, rows=-1) == 1
    assert q(nv, ldx=16) == 1                      # ldx < cols
    assert q(nv, x=None) == 1
    assert q(nv, codes=None) == 1
    assert q(nv, scales=None) == 1
    assert q(nv, g=None) == 1
    assert q(nv, x=MIS) == 1                       # misaligned input
    assert q(nv, ldx=36) == 1                      # row pitch not a multiple of 16 B
    assert q(nv, dt=7) == 1
    assert q(nv, mode=5) == 1
    assert q(nv, mode=0) == 3                      # per-tensor needs a workspace
    assert q(nv, mode=0, ws=A16, wsb=1) == 3       # too small
    assert q(nv, rows=1 << 27, cols=1 << 10, ldx=1 << 10) == 2   # too many blocks
    assert nv.lib.nvfp4_quantize_workspace_size(4096, 5120, 0) >= 4
    assert nv.lib.nvfp4_quantize_workspace_size(4096, 5120, 2) == 0


def test_quantize_no_alloc_argument_errors(nv):
    # The same host-side checks as nvfp4_quantize, without a workspace argument.
    def qn(x=A16, dt=1, rows=4, cols=32, ldx=32, codes=A16, scales=A16, g=A16, mode=0):
        return nv.lib.nvfp4_quantize_no_alloc(x, dt, rows, cols, ldx, codes, scales, g, mode, None)
    assert qn(cols=24, ldx=24) == 1
    assert qn(rows=-1) == 1
    assert qn(ldx=16) == 1
    assert qn(x=None) == 1
    assert qn(g=None) == 1
    assert qn(x=MIS) == 1
    assert qn(dt=7) == 1
    assert qn(mode=5) == 1
    assert qn(rows=1 << 27, cols=1 << 10, ldx=1 << 10) == 2


def g(nv, M=32, N=32, K=128, a=A16, sa=A16, ga=A16, pr=0, w=A16, sw=A16, gw=A16, y=A16, dt=1, ldy=32):
    return nv.lib.nvfp4_gemm(M, N, K, a, sa, ga, pr, w, sw, gw, y, dt, ldy, None, 0, None)


def test_gemm_argument_errors(nv):
    assert g(nv, K=24) == 1
    assert g(nv, K=0) == 1
    assert g(nv, M=-1) == 1
    assert g(nv, ldy=16) == 1
    assert g(nv, a=None) == 1
    assert g(nv, w=MIS) == 1
    assert g(nv, sa=MIS) == 1 and g(nv, sw=A16 + 4) == 1    # scales must be 16-byte aligned
    assert g(nv, gw=None) == 1
    assert g(nv, dt=3) == 1
    assert g(nv, pr=2) == 1
    assert g(nv, M=0) == 0 and g(nv, N=0, ldy=0) == 0     # empty products are no-ops


def test_decode_linear_argument_errors(nv):
    def d(N=32, K=128, x=A16, dt=1, mode=0, c=A16, s=A16, gl=A16, w=A16, sw=A16, gw=A16, y=A16, ydt=1):
        return nv.lib.nvfp4_decode_linear(N, K, x, dt, mode, c, s, gl, w, sw, gw, y, ydt, None)
    assert d(K=24) == 1 and d(K=0) == 1 and d(N=-1) == 1
    assert d(x=None) == 1 and d(x=MIS) == 1
    assert d(c=None) == 1 and d(c=A16 + 8) == 1 and d(s=A16 + 4) == 1   # codes, scales 16-byte aligned
    assert d(gl=None) == 1
    assert d(w=None) == 1 and d(sw=MIS) == 1 and d(gw=None) == 1 and d(y=None) == 1
    assert d(dt=7) == 1 and d(ydt=3) == 1 and d(mode=5) == 1


def test_fused_argument_errors(nv):
    widths = (ctypes.c_int64 * 3)(16, 0, 16)
    f = nv.lib.nvfp4_gemm_fused_segments
    assert f(32, 128, A16, A16, A16, 0, 3, ctypes.cast(widths, ctypes.c_void_p), A16, A16, A16, A16, 1, 48,
             None, 0, None) == 1                   # zero-width segment
    assert f(32, 128, A16, A16, A16, 0, 0, None, A16, A16, A16, A16, 1, 48, None, 0, None) == 1
    many = (ctypes.c_int64 * 65)(*([16] * 65))
    assert f(32, 128, A16, A16, A16, 0, 65, ctypes.cast(many, ctypes.c_void_p), A16, A16, A16, A16, 1,
             1040, None, 0, None) == 2
    ok = (ctypes.c_int64 * 2)(16, 16)
    assert f(32, 128, A16, A16, A16, 0, 2, ctypes.cast(ok, ctypes.c_void_p), A16, A16, A16, A16, 1, 16,
             None, 0, None) == 1                   # ldy < sum of widths


def test_fastdiv_host_logic(tmp_path):
    # The flat block index of the encoder is split into (row, block) with a multiply-high
    # division; check it on the host against integer division.
    src = tmp_path / "fd.cpp"
    src.write_text(
        '#include "nvfp4_internal.h"\n#include <cstdio>\nint main(){unsigned long long bad=0;\n'
        'unsigned ds[]={1,2,3,5,7,16,20,64,320,1088,1089,4095,65537,1000003,2147483647u,4294967295u};\n'
        'for(unsigned d: ds){auto f=nvfp4::make_fastdiv(d); unsigned long long x=88172645463325252ull;\n'
        ' for(long i=0;i<2000000;i++){x^=x<<13;x^=x>>7;x^=x<<17; unsigned n=(unsigned)x; if(i<1000) n=i;\n'
        '  if(i>=1000&&i<2000) n=0xFFFFFFFFu-(unsigned)(i-1000);\n'
        '  if(nvfp4::fastdiv(n,f)!=n/d) bad++;}}\nprintf("%llu\\n",bad); return bad!=0;}\n')
    exe = tmp_path / "fd"
    inc = os.path.join(ROOT, "nvfp4_w4a4_block_amd", "csrc")
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-O1", "-x", "hip", "--cuda-host-only", "-I", inc, str(src), "-o",
                        str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    """The GEMM source's generated gfx950 device assembly."""
    from nvfp4_w4a4_block_amd import build as b
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    r = subprocess.run([b.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
                        os.path.join(b.CSRC, "gemm.hip"), "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_m0_is_only_set_for_lds_copies(gemm_asm):
    """The GEMM's direct-to-LDS copies set M0 in inline assembly, which the compiler cannot be
    told about.  Check on the generated gfx950 assembly that every M0 write is one of those
    copies (immediately followed by its global_load_lds) and that nothing else reads M0."""
    from nvfp4_w4a4_block_amd import build as b
    assert b.check_m0(gemm_asm) > 0
    # the check rejects a stray M0 use and a copy without its own M0 write
    with pytest.raises(RuntimeError):
        b.check_m0("s_mov_b32 m0, s4\nglobal_load_lds_dwordx4 v1, off\ns_add_u32 s0, m0, 1\n")
    with pytest.raises(RuntimeError):
        b.check_m0("s_mov_b32 m0, s4\nglobal_load_lds_dwordx4 v1, off\nglobal_load_lds_dwordx4 v2, off\n")


def _kernel(name, body):
    return f"{name}:\n" + "\n".join("\t" + l if not l.startswith(".LBB") else l for l in body) + "\n.Lfunc_end0:\n"


def test_lds_refills_wait_for_reads(gemm_asm):
    """A direct-to-LDS copy writes LDS when its data arrives, so an LDS read of the bytes it
    overwrites must be complete before the copy is issued.  On the generated assembly, over
    every path through each kernel's branches: no copy is issued with an LDS read in flight,
    except the batch-1 kernel's read-ahead of its next item (6 reads, from another ring slot)."""
    from nvfp4_w4a4_block_amd import build as b
    found = b.check_lds_refills(gemm_asm)
    gemv = {k: v for k, v in found.items() if "gemm_gemv_kernel" in k}
    assert len(gemv) == 2 and all(v == 6 for v in gemv.values()), gemv
    others = {k: v for k, v in found.items() if k not in gemv}
    assert len(others) >= 10 and not any(others.values()), others

    count = lambda body: b.lds_reads_in_flight_at_copies(_kernel("k", body))["k"]
    copy = "global_load_lds_dword v2, s[0:1]"
    # straight line: a pending read counts, a wait retires it
    assert count(["ds_read_b32 v0, v1", copy, "s_endpgm"]) == 1
    assert count(["ds_read_b32 v0, v1", "s_waitcnt lgkmcnt(0)", copy, "s_endpgm"]) == 0
    # LDS operations retire in order: lgkmcnt(1) leaves only the newest in flight
    assert count(["ds_read_b32 v0, v1", "ds_read_b32 v3, v1", "s_waitcnt lgkmcnt(1)", copy, "s_endpgm"]) == 1
    assert count(["ds_read_b32 v0, v1", "ds_write_b32 v1, v0", "s_waitcnt lgkmcnt(1)", copy, "s_endpgm"]) == 0
    # a scalar load may complete first, so it does not stand in for the read
    assert count(["ds_read_b32 v0, v1", "s_load_dword s4, s[0:1], 0x0", "s_waitcnt lgkmcnt(1)", copy,
                  "s_endpgm"]) == 1
    # a branch that skips the wait, and a read carried round a loop to the copy at its top
    assert count(["ds_read_b32 v0, v1", "s_cbranch_scc1 .LBB0_2", "s_waitcnt lgkmcnt(0)", ".LBB0_2:", copy,
                  "s_endpgm"]) == 1
    assert count([".LBB0_1:", copy, "ds_read_b32 v0, v1", "s_cbranch_scc1 .LBB0_1", "s_endpgm"]) >= 1
    assert count([".LBB0_1:", copy, "ds_read_b32 v0, v1", "s_waitcnt lgkmcnt(0)", "s_cbranch_scc1 .LBB0_1",
                  "s_endpgm"]) == 0
    with pytest.raises(RuntimeError):
        b.check_lds_refills(_kernel("k", ["ds_read_b32 v0, v1", copy, "s_endpgm"]))
    b.check_lds_refills(_kernel("gemm_gemv_kernel_x", ["ds_read_b32 v0, v1", copy, "s_endpgm"]))


def test_nvfp4_out_argument_errors(nv):
    f = nv.lib.nvfp4_gemm_nvfp4_out
    w16 = (ctypes.c_int64 * 1)(16)
    w40 = (ctypes.c_int64 * 1)(40)

    def call(M=32, K=256, widths=w16, n=1, gy=A16, yc=A16, ys=A16):
        return f(M, K, A16, A16, A16, 0, n, ctypes.cast(widths, ctypes.c_void_p), A16, A16, A16, gy, yc, ys, None)

    assert call(widths=w40) == 1                   # N not a multiple of 16
    assert call(gy=None) == 1 and call(yc=None) == 1 and call(ys=A16 + 8) == 1
    assert call(K=272) == 2                        # K not a multiple of 128: no kernel takes it
    assert call(M=32, K=384) == 2                  # M > 16 needs K % 256 == 0
    assert call(M=1, K=1 << 24) == 2 and call(M=32, K=1 << 24) == 2   # K >= 2^24: only the plain kernel
    assert call(M=0) == 0                          # empty product: a no-op


def test_fp8_kv_argument_errors(nv):
    q, d = nv.lib.nvfp4_fp8_kv_quantize, nv.lib.nvfp4_fp8_kv_dequantize
    assert q(A16, 1, -1, A16, A16, None) == 1 and q(A16, 7, 16, A16, A16, None) == 1
    assert q(MIS, 1, 16, A16, A16, None) == 1 and q(A16, 1, 16, None, A16, None) == 1
    assert q(A16, 1, 16, A16, A16 + 4, None) == 1          # q must be 8-byte aligned
    assert d(A16, 16, A16, A16 + 8, 1, None) == 1          # y must be 16-byte aligned
    assert d(A16, 16, A16, A16, 5, None) == 1
    assert q(None, 1, 0, None, None, None) == 0 and d(None, 0, None, None, 0, None) == 0


def test_gdn_gates_argument_errors(nv):
    f = nv.lib.nvfp4_gemm_fused_gdn_gates
    w3 = (ctypes.c_int64 * 3)(64, 48, 48)
    w_uneq = (ctypes.c_int64 * 3)(64, 48, 32)
    w1 = (ctypes.c_int64 * 1)(48)

    def call(M=32, K=256, widths=w3, n=3, al=A16, dt=A16, gg=A16, beta=A16, y=A16):
        return f(M, K, A16, A16, A16, 0, n, ctypes.cast(widths, ctypes.c_void_p), A16, A16, A16, y, 1, 160,
                 al, dt, gg, beta, None, 0, None)

    assert call(widths=w_uneq) == 1                # the two gate segments differ in width
    assert call(widths=w1, n=1) == 1               # fewer than two segments
    assert call(al=None) == 1 and call(dt=None) == 1 and call(gg=None) == 1 and call(beta=None) == 1
    assert call(gg=A16 + 2) == 1 and call(beta=A16 + 1) == 1 and call(al=A16 + 2) == 1
    assert call(y=None) == 1
    assert call(M=0) == 0                          # empty product: a no-op


def test_swiglu_argument_errors(nv):
    f = nv.lib.nvfp4_gemm_swiglu

    def call(M=32, F=64, K=256, h=A16, dt=1, ldh=64, hg=A16, hc=A16, hs=A16, wg=A16):
        return f(M, F, K, A16, A16, A16, 0, A16, A16, wg, h, dt, ldh, hg, hc, hs, None)

    assert call(F=40) == 1 and call(F=0) == 1      # F not a positive multiple of 16
    assert call(h=None, hg=None, hc=None, hs=None) == 1     # no output asked for
    assert call(hg=None) == 1 and call(hc=None) == 1 and call(hs=None) == 1   # partial NVFP4 output
    assert call(hc=A16 + 8) == 1 and call(hs=A16 + 4) == 1 and call(hg=A16 + 2) == 1
    assert call(ldh=48) == 1 and call(dt=7) == 1 and call(h=A16 + 1) == 1
    assert call(wg=None) == 1
    assert call(K=272) == 2                        # K not a multiple of 128: no kernel takes it
    assert call(K=384) == 2                        # M > 16 needs K % 256 == 0
    assert call(M=0) == 0                          # empty product: a no-op
    g = nv.lib.nvfp4_interleave_gate_up
    assert g(40, 256, A16, A16, A16, A16, A16, A16, None) == 1      # F not a multiple of 16
    assert g(64, 40, A16, A16, A16, A16, A16, A16, None) == 1       # K not a multiple of 16
    assert g(64, 256, A16, A16, None, A16, A16, A16, None) == 1
    assert g(64, 256, A16, A16, A16, A16, A16, None, None) == 1


def test_mxfp4_argument_errors(nv):
    r = nv.lib.nvfp4_to_mxfp4
    assert r(4, 48, A16, A16, A16, A16, None) == 1            # cols not a multiple of 32
    assert r(-1, 64, A16, A16, A16, A16, None) == 1
    assert r(4, 64, A16 + 8, A16, A16, A16, None) == 1        # codes must be 16-byte aligned
    assert r(4, 64, A16, A16 + 1, A16, A16, None) == 1        # scales 2-byte aligned
    assert r(4, 64, A16, A16, None, A16, None) == 1
    assert r(0, 64, None, None, None, None, None) == 0
    g = nv.lib.nvfp4_mxfp4_gemm
    w = (ctypes.c_int64 * 1)(64)

    def call(M=32, K=512, y=A16, dt=1):
        return g(M, K, A16, A16, A16, 0, 1, ctypes.cast(w, ctypes.c_void_p), A16, A16, A16, y, dt, 64, None)

    assert call(K=384) == 2                        # K not a multiple of 256
    assert call(K=40) == 1                         # K not a multiple of 16
    assert call(y=None) == 1 and call(dt=7) == 1
    assert call(M=0) == 0


def test_header_is_c99_and_links_from_c(nv, tmp_path):
    """The header is plain C: a C99 program that takes the address of every declared entry point
    compiles with -pedantic -Werror, links against the library, and runs its host-only paths
    (version, status strings, argument errors detected before any launch)."""
    fns = _declared_functions()
    src = tmp_path / "abi_check.c"
    src.write_text("""#include <stdio.h>
#include "nvfp4.h"
typedef void (*fn_t)(void);
static const fn_t entry_points[] = {
""" + ",\n".join(f"  (fn_t){f}" for f in fns) + """
};
int main(void) {
  unsigned i;
  for (i = 0; i < sizeof entry_points / sizeof entry_points[0]; ++i)
    if (!entry_points[i]) return 1;
  if (nvfp4_version() <= 0) return 2;
  if (!nvfp4_status_string(NVFP4_ERR_INVALID_ARG)) return 3;
  /* K not a multiple of 16: rejected on the host, before anything touches a GPU */
  if (nvfp4_gemm(16, 16, 24, 0, 0, 0, 0, 0, 0, 0, 0, NVFP4_BF16, 16, 0, 0, 0) != NVFP4_ERR_INVALID_ARG) return 4;
  printf("ok %u\\n", (unsigned)(sizeof entry_points / sizeof entry_points[0]));
  return 0;
}
""")
    lib_dir = os.path.dirname(nv.library_path())
    exe = tmp_path / "abi_check"
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe), "-L", lib_dir, "-lnvfp4", f"-Wl,-rpath,{lib_dir}",
                        f"-Wl,-rpath-link,{rocm_lib}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == f"ok {len(fns)}", (r.returncode, r.stdout, r.stderr[-2000:])
