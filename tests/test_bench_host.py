"""bench.py's host-side parts: the command line contract and the oracle's
CPU baseline leg.  CPU only."""
import subprocess
import sys
from pathlib import Path

import bench
import workloads as W

ROOT = Path(__file__).resolve().parents[1]


def test_cpu_baseline_reports_all_threads_and_one():
    b = W.make_batch("tiny")
    r = bench.cpu_baseline(b, W.decode_kv_bytes(b)["logical"], 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["cores"] >= 1
    one = r["single_thread"]
    assert one["cores"] == 1 and one["value"] > 0
    assert "kv append" in r["sample"] and "one thread" in one["sample"]


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
