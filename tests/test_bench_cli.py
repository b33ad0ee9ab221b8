"""The benchmark's command line on the CPU: it measures one GPU, so a request
for more exits with a message before touching any device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_bench_lists_the_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0
    for name in ("mid_bf16", "dsv3_shard", "maverick_shard", "dedup_redundant",
                 "dsv3_ep8_receive", "tiny_fp32"):
        assert name in r.stdout
