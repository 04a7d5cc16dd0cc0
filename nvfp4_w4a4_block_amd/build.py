"""Build ``libnvfp4.so`` (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Run ``python nvfp4_w4a4_block_amd/build.py`` (as a script: importing the package would load the
library this builds).  The library lands next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4.so")
SOURCES = ["api.hip", "device.hip", "quantize.hip", "gemm.hip", "kv_fp8.hip", "mxfp4.hip"]
# The measurement script's calibration kernels (streaming read, copy, MFMA loop): a library of
# their own, outside the hot path's C ABI.
CALIB_LIB = os.path.join(HERE, "libnvfp4_calib.so")
CALIB_SOURCES = ["calibration.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Binary32 arithmetic exactly as written: no contraction into FMA, no fast math,
    # denormals kept, IEEE division.
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    # No packed fp32 instructions in generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd: list[str], verbose: bool) -> subprocess.CompletedProcess:
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def _stderr(res: subprocess.CompletedProcess) -> str:
    # hipcc's host pass warns about the device-only target feature; keep other output.
    return "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)


def check_m0(asm: str) -> int:
    """The GEMM's direct-to-LDS copies set M0 from inline assembly, which cannot tell the
    compiler that M0 changes.  Check on the generated gfx950 assembly that every M0 write is one
    of those copies (immediately followed by its global_load_lds), that nothing else touches M0
    and that every global_load_lds follows its own M0 write.  Returns the number of copies;
    raises RuntimeError otherwise."""
    import re
    code = [l.strip() for l in asm.splitlines()]
    code = [l for l in code if l and not l.startswith((";", "."))]
    writes = 0
    for i, l in enumerate(code):
        if not re.search(r"\bm0\b", l):
            continue
        if not re.fullmatch(r"s_mov_b32 m0, s\d+", l):
            raise RuntimeError(f"M0 used outside the LDS copies: {l}")
        if i + 1 >= len(code) or not code[i + 1].startswith("global_load_lds_dword"):
            raise RuntimeError(f"M0 write not followed by its copy: {l}")
        writes += 1
    loads = [i for i, l in enumerate(code) if l.startswith("global_load_lds")]
    if not writes or any(not code[i - 1].startswith("s_mov_b32 m0,") for i in loads):
        raise RuntimeError("a global_load_lds does not follow its own M0 write")
    return writes


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (each carries its own gfx950 code
    object), then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, os.pardir, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(HERE, os.pardir, "include")]
    def obj(src):
        return os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    objs = [obj(s) for s in SOURCES]
    calib_objs = [obj(s) for s in CALIB_SOURCES]
    cmds = [[hipcc(), *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", obj(s)]
            for s in SOURCES + CALIB_SOURCES]
    # The GEMM's device assembly, for the M0 check below.
    gemm_s = os.path.join(objdir, "gemm.s")
    cmds.append([hipcc(), *HIPCC_FLAGS, *inc, "--cuda-device-only", "-S", os.path.join(CSRC, "gemm.hip"),
                 "-o", gemm_s])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
        results = list(pool.map(lambda c: _run(c, verbose), cmds))
    for cmd, res in zip(cmds, results):
        err = _stderr(res)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}) on {cmd[-3]}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    with open(gemm_s) as f:
        check_m0(f.read())
    for lib, o in ((LIB, objs), (CALIB_LIB, calib_objs)):
        tmp = lib + ".tmp"
        res = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *o, "-o", tmp], verbose)
        if res.returncode != 0:
            raise RuntimeError(f"link of {os.path.basename(lib)} failed ({res.returncode}):\n{_stderr(res)}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
