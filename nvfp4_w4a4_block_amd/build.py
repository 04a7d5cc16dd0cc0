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


def lds_reads_in_flight_at_copies(asm: str) -> dict:
    """For each kernel of a gfx950 assembly listing that issues direct-to-LDS copies
    (global_load_lds): the largest number of LDS reads that may still be in flight when such a
    copy is issued, over every path through the kernel's branches.  A copy lands in LDS
    asynchronously, so a read of the bytes it overwrites must be complete before it is issued.

    Model: LDS instructions complete in issue order; scalar memory loads also count in lgkmcnt
    but complete in any order, so `s_waitcnt lgkmcnt(N)` is taken to retire them first (the
    case that leaves the most LDS reads in flight) and then the oldest LDS operations until at
    most N remain.  Only the newest 64 operations are tracked: a wait keeps at most its
    newest 15 (the counter is 4 bits wide), so older ones never change a result.  Returns
    {kernel symbol: count}."""
    import re
    result = {}
    funcs, cur = [], None
    for raw in asm.splitlines():
        m = re.match(r"^([A-Za-z_][\w.$]*):", raw)
        if m:
            cur = [m.group(1), []]
            funcs.append(cur)
            continue
        if cur is None:
            continue
        if raw.startswith(".Lfunc_end"):
            cur = None
            continue
        line = raw.split(";")[0].strip()
        if line:
            cur[1].append(line)
    for name, lines in funcs:
        if not any(l.startswith("global_load_lds") for l in lines):
            continue
        # basic blocks: a label starts one, a branch or s_endpgm ends one
        blocks, labels, blk = [], {}, []
        for l in lines:
            lm = re.match(r"^(\.L\w+):", l)
            if lm:
                if blk:
                    blocks.append(blk)
                    blk = []
                labels[lm.group(1)] = len(blocks)
                continue
            if l.startswith("."):
                continue
            blk.append(l)
            if l.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
                blocks.append(blk)
                blk = []
        if blk:
            blocks.append(blk)
        # successors of block i: a branch target (a label maps to the block that follows it)
        # and, unless the block ends in an unconditional branch or the end of the program, the
        # next block
        def succ(i):
            last = blocks[i][-1] if blocks[i] else ""
            op = last.split()[0] if last else ""
            out = []
            if op in ("s_endpgm", "s_setpc_b64"):
                return out
            if op.startswith(("s_branch", "s_cbranch")):
                tgt = last.split()[-1]
                if tgt not in labels:
                    raise RuntimeError(f"{name}: branch to unknown label {tgt}")
                out.append(labels[tgt])
                if op == "s_branch":
                    return [t for t in out if t < len(blocks)]
            if i + 1 < len(blocks):
                out.append(i + 1)
            return [t for t in out if t < len(blocks)]

        def step(q, l):
            op = l.split()[0]
            if op.startswith("ds_"):
                return q + ("r" if op.startswith("ds_read") else "o",)
            if op.startswith(("s_load", "s_buffer_load", "s_memtime", "s_memrealtime", "s_sendmsg")):
                return q + ("s",)
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", l)
                if m:
                    n = int(m.group(1))
                    q = list(q)
                    while len(q) > n:
                        if "s" in q:
                            q.remove("s")
                        else:
                            q.pop(0)
                    return tuple(q)
            return q

        # every (block, operations in flight at its entry) reachable from the kernel's entry
        seen = {(0, ())}
        work, worst = [(0, ())], 0
        while work:
            i, q = work.pop()
            for l in blocks[i]:
                if l.startswith("global_load_lds"):
                    worst = max(worst, q.count("r"))
                q = step(q, l)[-64:]
            for t in succ(i):
                if (t, q) not in seen:
                    seen.add((t, q))
                    if len(seen) > 100000:
                        raise RuntimeError(f"{name}: too many paths to follow")
                    work.append((t, q))
        result[name] = worst
    return result


# LDS reads allowed in flight at a direct-to-LDS copy, per kernel: none, except where a kernel
# reads the next ring slot ahead while it refills another one (the batch-1 kernel's next item:
# one 16-byte code read, one scale read and four token reads).
LDS_READ_AHEAD = {"gemm_gemv_kernel": 6}


def check_lds_refills(asm: str) -> dict:
    """Raise RuntimeError if any kernel may issue a direct-to-LDS copy while more LDS reads
    are in flight than LDS_READ_AHEAD allows it; returns the per-kernel counts."""
    found = lds_reads_in_flight_at_copies(asm)
    for fn, n in found.items():
        allowed = next((v for k, v in LDS_READ_AHEAD.items() if k in fn), 0)
        if n > allowed:
            raise RuntimeError(f"{fn}: a direct-to-LDS copy may be issued with {n} LDS reads in flight "
                               f"(at most {allowed} allowed)")
    return found


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
        text = f.read()
    check_m0(text)
    check_lds_refills(text)
    for lib, o in ((LIB, objs), (CALIB_LIB, calib_objs)):
        tmp = lib + ".tmp"
        res = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *o, "-o", tmp], verbose)
        if res.returncode != 0:
            raise RuntimeError(f"link of {os.path.basename(lib)} failed ({res.returncode}):\n{_stderr(res)}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
