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


# ------------------------------------------------ byte-counter summary guards
def _write_csv(folder, counter, kernel, value):
    import os
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "x_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        f.write(f'"{kernel}",{counter},{value}\n')


def test_pmc_means_requires_exactly_one_counter_file(tmp_path):
    import pytest
    d = tmp_path / "run"
    _write_csv(str(d / "a"), "FETCH_SIZE", "k", 1.0)
    assert bench._pmc_means(str(d), "FETCH_SIZE") == {"k": 1.0}
    _write_csv(str(d / "b"), "FETCH_SIZE", "k", 2.0)
    with pytest.raises(SystemExit, match="2 counter_collection"):
        bench._pmc_means(str(d), "FETCH_SIZE")


def test_summary_refuses_other_sources_and_unknown_kernels(tmp_path):
    import pytest
    known = sorted(k for k in bench.library_kernels() if "decode" in k)
    assert known, "the built library holds decode kernels"
    dirs = [str(tmp_path / n) for n in ("f", "w", "cf", "cw")]
    copy = "__amd_rocclr_copyBuffer"
    _write_csv(dirs[2], "FETCH_SIZE", copy, 524288.0)
    _write_csv(dirs[3], "WRITE_SIZE", copy, 1048576.0)
    # a folder never stamped at measurement time
    _write_csv(dirs[0], "FETCH_SIZE", known[0], 10.0)
    _write_csv(dirs[1], "WRITE_SIZE", known[0], 1.0)
    with pytest.raises(SystemExit, match="source_stamp"):
        bench.summarize_pmc("tiny", *dirs)
    # stamped, but on other decode sources
    for d in dirs[:2]:
        with open(f"{d}/{bench.STAMP}", "w") as f:
            f.write("decode_source_sha256_16: 0000000000000000\n")
    with pytest.raises(SystemExit, match="measured on decode sources"):
        bench.summarize_pmc("tiny", *dirs)
    # current sources, but a kernel the library no longer holds
    for d in dirs[:2]:
        bench.stamp_source(d)
    gone = "void pkv::decode_gqa8_mfma_kernel<128, 32>(pkv::DecodeParams)"
    _write_csv(dirs[0], "FETCH_SIZE", gone, 10.0)
    with pytest.raises(SystemExit, match="not in the current library"):
        bench.summarize_pmc("tiny", *dirs)


def test_measurement_helpers_are_built_and_exported():
    import shutil
    lib = Path(bench.BENCH_LIB)
    assert lib.exists(), "build() makes libpkv_bench.so"
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", str(lib)], capture_output=True, text=True).stdout
        assert " T pkvb_stream_read" in out
        assert " T pkvb_mfma_rate" in out
