"""Host logic of bench.py, without a GPU: the one-GPU contract, the source digest that ties stored
HBM byte counts to the GEMM's code, and the CPU-baseline record of the oracle."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_digest_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) { return x + 1; }\n")
    b.write_text("// leading comment\nint f(int x)  {\n  /* block\n comment */ return x + 1;  // tail\n}\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    assert bench.source_digest([str(a)]) != bench.source_digest([str(c)])


def test_cpu_baseline_record():
    small_decode = workloads.Decode(N=64, K=512)
    r = bench.cpu_baseline(workloads.TINY, sample_rows=16, decode_m=4, d=small_decode)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1 and r["host_cores"] >= 1
    assert "16 of 16 rows" in r["sample"]
    assert r["quantize"]["gbs"] > 0 and r["quantize"]["threads"] == 1
    assert r["decode"]["gbs"] > 0 and "M = 4" in r["decode"]["sample"]
