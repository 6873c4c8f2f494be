"""Builds libpkv.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Each .hip file is compiled to an object in parallel, then linked into a
shared library next to this file.  Packed-fp32 instructions are disabled
(-packed-fp32-ops); the host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

HERE = Path(__file__).resolve().parent
ROOT = HERE.parent
CSRC = HERE / "csrc"
BUILD = HERE / "_build"
LIB = HERE / "libpkv.so"
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", str(ROOT / "include"), "-I", str(CSRC)]


# Per-source options.  decode.hip: MFMA accumulators in ordinary VGPRs (the
# grouped-query decode rescales and stores them with vector ALU code every
# step, which otherwise copies them between AGPRs and VGPRs around each
# MFMA).
SOURCE_FLAGS = {"decode.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _compile(src: Path, verbose: bool) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src.name, []), "-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))
    jobs = jobs or min(len(srcs), os.cpu_count() or 1, 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", str(tmp),
           *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


# Measurement helpers, apart from the library: a streaming-read kernel that
# bench.py times as the reference for a plain sequential read of HBM, and
# MFMA-only kernels, the reference for what the matrix cores sustain.
BENCH_SRCS = [CSRC / "bench" / "stream_read.hip", CSRC / "bench" / "mfma_rate.hip"]
BENCH_LIB = HERE / "libpkv_bench.so"


def build_bench(verbose: bool = False) -> Path:
    tmp = BENCH_LIB.with_suffix(".so.tmp")
    # accumulators of the MFMA-only kernels in VGPRs, as the prefill keeps them
    cmd = [hipcc(), *FLAGS, "-mllvm", "--amdgpu-mfma-vgpr-form", "-shared", "-o", str(tmp),
           *map(str, BENCH_SRCS)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        raise RuntimeError(f"hipcc failed on the measurement helpers:\n{err}")
    os.replace(tmp, BENCH_LIB)
    return BENCH_LIB


# Host-only build of the plain host sources with AddressSanitizer and
# UndefinedBehaviorSanitizer (g++, no device code): the block manager, the
# scheduler, the precondition checks and the status strings.  The binding
# takes them from it when $PKV_HOST_LIB names it; load it with libasan
# preloaded.
HOST_SOURCES = ("block_manager.cpp", "scheduler.cpp", "validate.cpp")
HOST_SAN_LIB = HERE / "libpkv_host_asan.so"
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]


def build_host_sanitized(verbose: bool = False) -> Path:
    cmd = ["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", *SANITIZE,
           "-I", str(ROOT / "include"), "-o", str(HOST_SAN_LIB),
           *(str(CSRC / f) for f in HOST_SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return HOST_SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_bench(verbose=True)
