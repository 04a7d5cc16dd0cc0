"""Host-side replay of the copy and wait schedule shared by the K-split decode kernels
(gemm_decode_lds_kernel, the 4 x 4 x 4 small-batch kernel and the MXFP4 gemm_mx_decode_lds_kernel
in csrc/gemm.hip).

Each wavefront streams its own range of 256-wide K stages through a private LDS ring of
kDlDepth stage slots, NC direct-to-LDS copies per stage (one per 1 KB chunk of rows it copies),
and the scale bytes in blocks of 8 stages (16 for the MXFP4 kernel, whose E8M0 bytes are half
as many) held in two buffers, NC copies per block.  Before it
reads stage t it waits until at most NC (kDlDepth - 1) copies are in flight.  Vector-memory
operations of a wavefront complete in issue order, so that wait leaves only the youngest
NC (kDlDepth - 1) copies outstanding.  The replay issues the copies in the kernels' order, for
every chunk count the kernels instantiate and every stage count a wavefront can get, and checks:
  * every read finds its stage's copies and its scale block's copies complete;
  * no copy targets a ring slot or scale buffer whose contents a later read still needs;
  * the wait is exact: one more copy in flight would leave some read's data outstanding.
The ring depth is read from the kernel source, so a change there is replayed as well."""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "nvfp4_w4a4_block_amd", "csrc", "gemm.hip")


def _depth() -> int:
    m = re.search(r"constexpr int kDlDepth = (\d+);", open(SRC).read())
    assert m, "kDlDepth not found in gemm.hip"
    return int(m.group(1))


def _replay(nc: int, cnt: int, depth: int, allowed: int, block: int = 8):
    """Replay one wavefront with cnt stages; return the first violation as a string, or None."""
    issued = []                 # copies in issue order: ("C", stage, chunk) or ("S", block, chunk)
    slot_stage = {}             # ring slot -> stage whose copy landed there last
    buf_block = {}              # scale buffer -> block whose copy landed there last
    done = 0                    # copies known complete (a prefix of `issued`, in-order completion)

    def copy_codes(t):
        slot = t % depth
        if slot in slot_stage and slot_stage[slot] < cnt and slot_stage[slot] > last_read[0]:
            return f"stage {t} overwrites slot {slot} before stage {slot_stage[slot]} is read"
        slot_stage[slot] = t
        issued.extend(("C", t, c) for c in range(nc))
        return None

    def copy_scales(b):
        buf = b & 1
        if buf in buf_block:
            old = buf_block[buf]
            if min(old * block + block - 1, cnt - 1) > last_read[0]:   # a stage of the old block is unread
                return f"scale block {b} overwrites block {old} before its stages are read"
        buf_block[buf] = b
        issued.extend(("S", b, c) for c in range(nc))
        return None

    last_read = [-1]
    err = copy_scales(0)
    for t in range(depth):
        err = err or copy_codes(t)
    if err:
        return err
    for t in range(cnt):
        done = max(done, len(issued) - allowed)            # the wait: at most `allowed` in flight
        complete = set(issued[:done])
        if any(("C", t, c) not in complete or ("S", t // block, c) not in complete for c in range(nc)):
            return f"stage {t} read with its copies in flight"
        if slot_stage.get(t % depth) != t or buf_block.get((t // block) & 1) != t // block:
            return f"stage {t} read from a slot or buffer holding other data"
        last_read[0] = t
        err = copy_codes(t + depth)
        if not err and (t + depth) % block == 0:
            err = copy_scales((t + depth) // block)
        if err:
            return err
    return None


# NC = W chunks + token chunks: the 4 x 4 x 4 kernel copies 2 + 1 or 3 + 1, the 16 x 16 x 32 and
# MXFP4 kernels 2..4 + 1..2.  The MXFP4 kernel's wavefronts take even stage counts.
@pytest.mark.parametrize("block", [8, 16])
@pytest.mark.parametrize("nc", [3, 4, 5, 6])
def test_waits_cover_every_read(nc, block):
    depth = _depth()
    for cnt in range(1, 80):
        err = _replay(nc, cnt, depth, nc * (depth - 1), block)
        assert err is None, f"NC={nc} stages={cnt} block={block}: {err}"


@pytest.mark.parametrize("block", [8, 16])
@pytest.mark.parametrize("nc", [3, 4, 5, 6])
def test_waits_are_exact(nc, block):
    depth = _depth()
    failures = [cnt for cnt in range(1, 80)
                if _replay(nc, cnt, depth, nc * (depth - 1) + 1, block) is not None]
    assert failures, f"NC={nc}: a wait allowing one more copy in flight never fails, so it is not exact"


def test_replay_catches_a_short_wait():
    # The replay itself: waiting for one stage fewer than the ring holds must be caught.
    depth = _depth()
    assert _replay(4, 20, depth, 4 * depth) is not None


def test_kernels_wait_as_replayed():
    # The three K-split decode kernels wait with the count the replay checks.
    src = open(SRC).read()
    assert src.count("vmcnt_imm(NC * (kDlDepth - 1))") == 3
