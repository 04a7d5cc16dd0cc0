"""Concurrent first calls: several host threads of a fresh process make their first
quantize + GEMM calls (and a one-call batch-1 decode) at the same moment, each on its own stream, so the library's once-per-
device set-up (kernel LDS limits, the compute-unit count, the static scratch address) runs
while other threads are already calling in.  Every thread's results must equal, bit for bit,
those of the same calls made afterwards by one thread.  The workers run in a child process so
that no earlier test has already set the device up."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import threading
import numpy as np
import torch
import nvfp4_w4a4_block_amd as nv
import workloads

dev = torch.device("cuda:0")
NT = 4
# Inputs are made with torch only; the library has not been called yet.
xs = [torch.from_numpy(workloads.activation(90, i, 512, 1024, outlier_frac=0.01)).to(dev).to(torch.bfloat16)
      for i in range(NT)]
ws = [torch.from_numpy(workloads.weight(90, 10 + i, 768, 1024)).to(dev).to(torch.bfloat16) for i in range(NT)]
xd = [x[:4].contiguous() for x in xs]
torch.cuda.synchronize()

def step(i):
    a = nv.quantize(xs[i])
    q = nv.quantize(ws[i])
    y = nv.gemm(a, q, torch.float32)                         # prefill kernel (M = 512)
    ad = nv.quantize(xd[i], "per_row")
    yd = nv.gemm(ad, q, torch.float32)                      # decode kernel (M = 4)
    y1, a1 = nv.decode_linear(xd[i][:1], q, out_dtype=torch.float32)   # batch 1, one launch
    return [a.codes, a.scales, a.global_scale, q.codes, q.scales, y, ad.codes, ad.scales, yd,
            a1.codes, a1.scales, a1.global_scale, y1]

results = [None] * NT
errors = []
go = threading.Barrier(NT)

def worker(i):
    try:
        s = torch.cuda.Stream(dev)
        with torch.cuda.stream(s):
            go.wait()
            out = step(i)
        s.synchronize()
        results[i] = [t.clone() for t in out]
    except BaseException as e:
        errors.append(repr(e))

threads = [threading.Thread(target=worker, args=(i,)) for i in range(NT)]
for t in threads:
    t.start()
for t in threads:
    t.join()
assert not errors, errors
# the same calls, one thread, the default stream
for i in range(NT):
    want = step(i)
    torch.cuda.synchronize()
    for j, (g, w) in enumerate(zip(results[i], want)):
        assert torch.equal(g.view(torch.uint8), w.view(torch.uint8)), (i, j)
print("threads ok")
'''


def test_concurrent_first_calls_from_threads():
    print("case: 4 threads, first quantize + GEMM calls at once, own streams", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": ROOT})
    assert r.returncode == 0 and "threads ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
