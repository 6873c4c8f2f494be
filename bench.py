#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the path over one batch: kv append of the step's new
rows, then paged decode (and, for the mixed workload, the causal prefill
chunks).  Inputs are seeded synthetic batches (workloads.py), resident in HBM
before timing starts.

Default run: the headline is the long-context workload (8 sequences x 32,768
tokens, 4 GiB of K/V per step, the largest single-GPU batch), and the same
measurement of the Llama-shaped decode, the mixed prefill + decode step and
the grouped-query batch with a shared prefix goes into ``per_config``.

Cold-cache timing: the batch is replicated R times in HBM (distinct pools,
queries and outputs) and consecutive steps rotate over the replicas, so the
bytes a step reads were last touched R-1 steps earlier -- far more than the
256 MB Infinity Cache holds (R = 1 when one step alone reads more than 2 GB).
One HIP graph holds R consecutive steps (one per replica, in rotation order)
and one graph per replica holds a single step; K steps replay the R-step
graph back to back, then single-step graphs for the remainder, bracketed by
synchronisations; ms_per_step is the event time / K.

Roofline of the dominant call (decode): algorithmic bytes per launch (KV rows
read once -- each physical (block, offset) once -- plus queries and outputs)
divided by its launch duration, against the 8 TB/s datasheet peak and, as
frac_of_stream_read, against a plain sequential read of 4 GiB timed the same
way on the same device (``stream_read``), and as frac_of_stream_read_same_bytes
against a read of the call's own byte count (cold windows of the same buffer),
which pays the same launch, ramp and drain as a call that short.  The mixed step's prefill FLOP rate
is likewise set against the 2.5 PFLOP/s datasheet figure and, as
frac_of_mfma_reference, against an MFMA-only kernel of the same instruction
(``mfma_reference``).  Durations come from HIP events on the
launch stream around batches of back-to-back calls (a spin kernel keeps the
GPU ahead of the host), divided by the batch size; the median over batches
is reported with its p10 / p90.  This does not depend on --steps.  The step
time itself is ms_per_step (K steps / K); its spread comes from batches of
back-to-back steps through the same graphs (step_us_median, step_us_p10,
step_us_p90).

CPU baseline: the CPU oracle (test infrastructure) timed on the host cores on
a bounded sample of the same batch's rows, median of 3 runs; the pool copy
the oracle needs is made before the clock starts.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, datasheet
METRIC = ("paged decode KV GB/s and % of HBM peak; seq-steps/s per batch on 1 MI355X")
HEADLINE = "long"
PER_CONFIG = ("llama_decode", "mixed", "gqa_shared")
# launch-duration batches: TIMING_BATCHES batches of TIMING_CALLS calls
TIMING_BATCHES = 10
TIMING_CALLS = 20


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=sorted(W.SPECS),
                    help=f"measure this workload alone (default: {HEADLINE} as the "
                         f"headline, with {', '.join(PER_CONFIG)} in per_config)")
    ap.add_argument("--per-config", default=None,
                    help="comma-separated workloads measured into per_config beside the "
                         "headline ('' for none)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough for cold caches")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="eager launches")
    ap.add_argument("--no-order", action="store_true",
                    help="dispatch decode sequences in batch order (default: the host "
                         "passes a longest-first order, as a serving loop that knows its "
                         "lengths does)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=9.0,
                    help="CPU time budget of the headline's oracle baseline (three runs); "
                         "per_config entries take a third of it each")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three plain 1 GiB device copies (the known-size "
                         "kernel that scales the HBM byte counters)")
    ap.add_argument("--stamp-source", metavar="DIR",
                    help="write the hash of the decode sources and of the built library "
                         "into DIR/source_stamp.txt (run right before profiling into DIR)")
    ap.add_argument("--block-size-sweep", action="store_true",
                    help="time the decode of the workload's batch at block sizes 1, 8, "
                         "16 and 32 (same lengths and pool capacity in tokens) and "
                         "print one JSON line per block size")
    ap.add_argument("--prefill-sweep", action="store_true",
                    help="time prefill alone on batches of few query tiles over long "
                         "prefixes (the key-range split) and on the mixed step's chunks")
    ap.add_argument("--swap-bench", action="store_true",
                    help="time swapping blocks of the workload's shape out to a pinned "
                         "host pool and back (kernel and DMA paths); one JSON line per "
                         "direction and path")
    ap.add_argument("--swap-blocks", type=int, default=1024)
    ap.add_argument("--serve", action="store_true",
                    help="multi-step continuous batching: the native scheduler drives "
                         "append / prefill / decode over many steps; prints one JSON line")
    ap.add_argument("--serve-requests", type=int, default=256)
    ap.add_argument("--serve-batch", type=int, default=32)
    ap.add_argument("--serve-tokens", type=int, default=2048)
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH",
                                                          "COPY_WRITE"),
                    help="turn four rocprofv3 --pmc output folders (FETCH_SIZE and "
                         "WRITE_SIZE of this workload's decode, then of the copy "
                         "calibration) into the traffic summary under profiles/")
    return ap.parse_args()


# --------------------------------------------------------------- HBM traffic
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SOURCES = ["paged_kv_cache_407_amd/csrc/decode.hip",
                  "paged_kv_cache_407_amd/csrc/common.hpp",
                  "paged_kv_cache_407_amd/csrc/kernels.hpp"]
LIB_FILE = os.path.join(ROOT, "paged_kv_cache_407_amd", "libpkv.so")
STAMP = "source_stamp.txt"
COPY_BYTES = 1 << 30


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _file_hash(path: str) -> str:
    h = hashlib.sha256()
    with open(path, "rb") as fh:
        for chunk in iter(lambda: fh.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()[:16]


def stamp_source(folder: str):
    """Records, at measurement time, which decode sources and which built
    library the counters in ``folder`` will come from."""
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, STAMP), "w") as f:
        f.write(f"decode_source_sha256_16: {decode_source_hash()}\n")
        f.write(f"libpkv_sha256_16: {_file_hash(LIB_FILE)}\n")
    log(f"stamped {folder}")


def _read_stamp(folder: str) -> dict:
    path = os.path.join(folder, STAMP)
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: profile into a folder stamped by "
                         f"bench.py --stamp-source right before the run")
    kv = {}
    for line in open(path):
        if ": " in line:
            k, v = line.split(": ", 1)
            kv[k.strip()] = v.strip()
    return kv


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, f"decode_{workload}_hbm_traffic.txt")


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"three copies of {COPY_BYTES} bytes done")


def _pmc_means(folder: str, counter: str) -> dict:
    """Mean counter value (KiB per dispatch) per kernel name, from the one
    counter CSV of a fresh rocprofv3 output folder."""
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"{folder} holds {len(files)} counter_collection.csv files; "
                         f"profile each pass into a fresh folder")
    vals = {}
    with open(files[0]) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows in {files[0]}")
    return {k: sum(v) / len(v) for k, v in vals.items()}


def library_kernels() -> set:
    """Demangled names of the kernels the current libpkv.so holds (their
    host launch stubs), in the form rocprofv3 reports them."""
    out = subprocess.run(["nm", "-C", LIB_FILE], capture_output=True, text=True,
                         check=True).stdout
    names = set()
    for line in out.splitlines():
        parts = line.split(" ", 2)
        if len(parts) == 3 and parts[1] in ("V", "D", "T", "W") and "pkv::" in parts[2]:
            names.add(parts[2])
    return names


def summarize_pmc(workload: str, fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """HBM bytes per decode call = FETCH_SIZE and WRITE_SIZE of its kernels,
    each scaled by (known bytes / counter reading) of a plain 1 GiB copy.
    Refuses counters taken from other decode sources, or naming kernels the
    current library does not hold."""
    cur = decode_source_hash()
    stamps = [_read_stamp(d) for d in (fetch_dir, write_dir)]
    for d, st in zip((fetch_dir, write_dir), stamps):
        if st.get("decode_source_sha256_16") != cur:
            raise SystemExit(f"{d} was measured on decode sources "
                             f"{st.get('decode_source_sha256_16')}, current is {cur}")
    fetch = _pmc_means(fetch_dir, "FETCH_SIZE")
    write = _pmc_means(write_dir, "WRITE_SIZE")
    cf = _pmc_means(cfetch_dir, "FETCH_SIZE")
    cw = _pmc_means(cwrite_dir, "WRITE_SIZE")
    copy_k = [k for k in cf if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy_k:
        raise SystemExit(f"no copy kernel among {list(cf)}")
    ck = max(copy_k, key=lambda k: cf[k])
    f_fetch = COPY_BYTES / (cf[ck] * 1024)
    f_write = COPY_BYTES / (cw[ck] * 1024)
    dec = sorted(k for k in fetch if "decode" in k)
    known = library_kernels()
    stale = [k for k in set(dec) | {k for k in write if "decode" in k} if k not in known]
    if stale:
        raise SystemExit(f"kernels not in the current library: {stale}")
    if not dec:
        raise SystemExit(f"no decode kernel in {fetch_dir}")
    lines = [f"# HBM traffic of one paged_attention_decode call, workload {workload}",
             f"decode_source_sha256_16: {cur}",
             f"libpkv_sha256_16 (measured): {stamps[0].get('libpkv_sha256_16')}",
             f"copy_kernel: {ck}",
             f"copy_bytes_read: {COPY_BYTES}",
             f"copy_FETCH_SIZE_KiB: {cf[ck]:.1f}",
             f"copy_WRITE_SIZE_KiB: {cw[ck]:.1f}",
             f"fetch_scale: {f_fetch:.4f}",
             f"write_scale: {f_write:.4f}"]
    tot_r = tot_w = 0.0
    for k in dec:
        r = fetch[k] * 1024 * f_fetch
        w = write.get(k, 0.0) * 1024 * f_write
        tot_r += r
        tot_w += w
        lines.append(f"kernel: {k} | FETCH_SIZE_KiB {fetch[k]:.1f} | WRITE_SIZE_KiB "
                     f"{write.get(k, 0.0):.1f} | read_bytes {r:.0f} | written_bytes {w:.0f}")
    b = W.make_batch(workload)
    kvb = W.decode_kv_bytes(b)
    kv = kvb["unique"] if b.spec.shared_prefix else kvb["logical"]
    alg = kv + b.q_dec.nbytes + b.num_dec * b.spec.num_q_heads * b.spec.head_dim * 4
    lines.append(f"traffic_bytes_per_call: {tot_r + tot_w:.0f}")
    lines.append(f"algorithmic_bytes_per_call: {alg}")
    lines.append(f"traffic_over_algorithmic: {(tot_r + tot_w) / alg:.4f}")
    lines.append("commands (from the repository root, TMPDIR=/tmp; each pass into a fresh "
                 "folder):")
    lines.append(f"  python3 bench.py --stamp-source <dir> && rocprofv3 --pmc FETCH_SIZE -f csv "
                 f"--kernel-include-regex pkv -d <dir> -- python3 bench.py --workload "
                 f"{workload} --steps 10 --warmup 2 --no-cpu-baseline --no-graph")
    lines.append("  (the same with WRITE_SIZE)")
    lines.append("  rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -- python3 bench.py "
                 "--copy-calibration   (and WRITE_SIZE)")
    lines.append(f"  python3 bench.py --workload {workload} --summarize-pmc "
                 "<fetch dir> <write dir> <copy fetch dir> <copy write dir>")
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(workload), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_traffic(workload: str):
    """Traffic per decode call from the committed summary, or None when there
    is none or the decode kernel has changed since it was measured."""
    try:
        kv = {}
        for line in open(traffic_path(workload)):
            if ": " in line and not line.startswith(("#", " ")):
                k, v = line.split(": ", 1)
                kv[k] = v.strip()
        if kv.get("decode_source_sha256_16") != decode_source_hash():
            return None
        return int(float(kv["traffic_bytes_per_call"]))
    except (OSError, KeyError, ValueError):
        return None


# ------------------------------------------------------------------- timing
def launch_stats(call, batches=TIMING_BATCHES, per_batch=TIMING_CALLS) -> dict:
    """Launch duration of call(i) on the current stream, in us: HIP events
    around each batch of per_batch back-to-back calls, divided by per_batch
    (the kernels' duration plus the gaps between them, as a profiler sees
    them), with a spin kernel keeping the GPU ahead of the host before every
    batch.  Median, mean, p10 and p90 over the batches."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(batches)]
    torch.cuda.synchronize()
    i = 0
    for e0, e1 in evs:
        torch.cuda._sleep(20_000_000)
        e0.record()
        for _ in range(per_batch):
            call(i)
            i += 1
        e1.record()
    torch.cuda.synchronize()
    d = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3 / per_batch
    return {"us_median": round(float(np.median(d)), 3), "us_mean": round(float(d.mean()), 3),
            "us_p10": round(float(np.percentile(d, 10)), 3),
            "us_p90": round(float(np.percentile(d, 90)), 3),
            "calls": batches * per_batch, "batches": batches}


STREAM_BYTES = 4 << 30
STREAM_GRIDS = (8192, 32768, 65536, 131072)
BENCH_LIB = os.path.join(ROOT, "paged_kv_cache_407_amd", "libpkv_bench.so")


MFMA_ITERS = 1024
MFMA_GRIDS = (256, 512, 1024, 2048)
MFMA_SHAPES = {"f16_16x16x32": (0, 16 * 16 * 32 * 2, 8), "f16_32x32x16": (1, 32 * 32 * 16 * 2, 4)}


def mfma_reference(dev) -> dict:
    """What the matrix cores sustain on this device: MFMA-only kernels of
    libpkv_bench.so (each wave issues independent accumulator chains of one
    fp16 shape and nothing else), timed like the prefill (launch_stats), best
    of a few grid sizes, per shape.  The prefill uses the 16x16x32 shape; its
    FLOP rate is also reported as a fraction of that shape's reference."""
    import ctypes
    import torch
    if not os.path.exists(BENCH_LIB):
        raise SystemExit(f"{BENCH_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(BENCH_LIB)
    fn = lib.pkvb_mfma_rate
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    out = torch.empty(max(MFMA_GRIDS) * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, (shape, flop_per_inst, chains) in MFMA_SHAPES.items():
        best = None
        for grid in MFMA_GRIDS:
            def call(_i, grid=grid, shape=shape):
                rc = fn(out.data_ptr(), shape, grid, MFMA_ITERS, 0.125, 0.125, stream)
                if rc:
                    raise RuntimeError(f"pkvb_mfma_rate failed: hip error {rc}")
            call(0)
            torch.cuda.synchronize()
            st = launch_stats(call, batches=5, per_batch=5)
            flops = grid * 4 * MFMA_ITERS * chains * flop_per_inst
            tf = flops / (st["us_median"] * 1e-6) / 1e12
            log(f"mfma {name}, {grid} workgroups: {st['us_median']} us, {tf:.1f} TFLOP/s")
            if best is None or tf > best["TFLOPs"]:
                best = {"TFLOPs": round(tf, 1), "frac_of_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                        "workgroups": grid, "us_median": st["us_median"],
                        "kernel": f"mfma{name[4:]}_kernel (libpkv_bench.so)"}
        res[name] = best
    del out
    torch.cuda.synchronize()
    return res


def stream_read_reference(dev, sizes=()) -> tuple[dict, dict]:
    """What a plain sequential read of HBM reaches on this device: the
    streaming-read kernel of libpkv_bench.so (16-byte nontemporal loads, the
    decode's load form; two streams, the halves of the buffer), timed like
    the decode (launch_stats), best of a few grid sizes.  First over a whole
    4 GiB buffer; then, for each byte count in `sizes`, over windows of that
    size taken in turn from the same buffer (each window last read 4 GiB
    earlier, so cold like the decode's replicas): a short call pays the
    same launch, ramp and drain as the decode call of that size.  Returns
    (the 4 GiB figure, {bytes: figure})."""
    import ctypes
    import torch
    if not os.path.exists(BENCH_LIB):
        raise SystemExit(f"{BENCH_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(BENCH_LIB)
    fn = lib.pkvb_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p]
    buf = torch.ones(STREAM_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def best_of(nbytes):
        windows = max(1, STREAM_BYTES // nbytes)
        best = None
        for grid in STREAM_GRIDS:
            def call(i, grid=grid):
                off = (i % windows) * nbytes
                rc = fn(buf.data_ptr() + off, nbytes, sink.data_ptr(), grid, stream)
                if rc:
                    raise RuntimeError(f"pkvb_stream_read failed: hip error {rc}")
            call(0)
            torch.cuda.synchronize()
            st = launch_stats(call, batches=5, per_batch=5)
            gbs = nbytes / (st["us_median"] * 1e-6) / 1e9
            log(f"stream read of {nbytes} B, {grid} workgroups: {st['us_median']} us, {gbs:.1f} GB/s")
            if best is None or gbs > best["GBps"]:
                best = {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                        "bytes": nbytes, "workgroups": grid, "us_median": st["us_median"],
                        "kernel": "stream_read_kernel (libpkv_bench.so)"}
        return best

    whole = best_of(STREAM_BYTES)
    per_size = {n: best_of(n) for n in sorted(set(sizes)) if 0 < n < STREAM_BYTES}
    del buf, sink
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return whole, per_size


def to_device(a, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.float16)
    return torch.from_numpy(a).to(dev)


# ------------------------------------------------------------- measurement
def measure(name: str, args, dev, cpu_seconds: float | None) -> dict:
    """One workload: K timed steps (append + prefill + decode) through HIP
    graphs over cold replicas, the decode's (and prefill's) launch durations,
    and the oracle baseline when cpu_seconds is given."""
    import torch
    import paged_kv_cache_407_amd as pkv

    t0 = time.time()
    b = W.make_batch(name)
    log(f"generated {name} in {time.time() - t0:.1f}s")
    spec = b.spec
    S = b.num_dec
    C = b.num_pf
    kvb = W.decode_kv_bytes(b)
    kv_bytes = kvb["unique"] if spec.shared_prefix else kvb["logical"]
    q_bytes = b.q_dec.nbytes if S else 0
    out_bytes = S * spec.num_q_heads * spec.head_dim * 4
    decode_alg_bytes = kv_bytes + q_bytes + out_bytes
    append_bytes = 2 * 2 * int((b.slot_mapping >= 0).sum()) * spec.num_kv_heads * spec.head_dim * 2
    pf_flops = W.prefill_flops(b)
    max_len = int(b.lens_dec.max()) if S else 1
    max_q = int(np.diff(b.cu_q_lens).max()) if C else 0
    max_len_pf = int(b.lens_pf.max()) if C else 1
    pf_ws_bytes = (pkv.prefill_workspace_size(C, int(b.cu_q_lens[-1]), max_q, spec.num_q_heads,
                                              spec.head_dim, max_len_pf) if C else 0)
    part = pkv.decode_partition_size(S, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                                     spec.block_size, max_len, args.partition_size)
    ws_bytes = pkv.decode_workspace_size(S, spec.num_q_heads, spec.num_kv_heads,
                                         spec.head_dim, spec.block_size, max_len,
                                         args.partition_size)

    touched = kv_bytes + append_bytes
    if C:
        touched += int(b.lens_pf.astype(np.int64).sum()) * W.kv_token_bytes(b)
    R = args.replicas or max(1, min(16, math.ceil(2.0e9 / max(touched, 1))))
    R = max(1, min(R, int(64e9 // b.nbytes_pool())))
    log(f"{name}: replicas {R}: pool {b.nbytes_pool() / 2**30:.2f} GiB each, "
        f"{touched / 1e6:.1f} MB touched per step; partition {part} tokens")

    to_dev = lambda a: to_device(a, dev)  # noqa: E731
    kc0, vc0 = to_dev(b.k_cache), to_dev(b.v_cache)
    reps = []
    for r in range(R):
        rep = {"kc": kc0 if r == 0 else kc0.clone(), "vc": vc0 if r == 0 else vc0.clone(),
               "nk": to_dev(b.new_k), "nv": to_dev(b.new_v)}
        if S:
            rep["q"] = to_dev(b.q_dec)
            rep["out"] = torch.empty((S, spec.num_q_heads, spec.head_dim), dtype=torch.float32,
                                     device=dev)
            rep["ws"] = (torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
                         if ws_bytes else None)
        if C:
            rep["qp"] = to_dev(b.q_pf)
            rep["outp"] = torch.empty(tuple(b.q_pf.shape), dtype=torch.float32, device=dev)
        reps.append(rep)
    slots = to_dev(b.slot_mapping)
    if S:
        tab, lens = to_dev(b.tables_dec), to_dev(b.lens_dec)
    if C:
        tabp, lensp, cu = to_dev(b.tables_pf), to_dev(b.lens_pf), to_dev(b.cu_q_lens)
        # one stream runs every step in turn: the replicas share it
        ws_pf = torch.empty(pf_ws_bytes, dtype=torch.uint8, device=dev) if pf_ws_bytes else None
    torch.cuda.synchronize()

    def do_append(rep):
        pkv.kv_append(rep["nk"], rep["nv"], rep["kc"], rep["vc"], slots)

    # the dispatch order, from the host's copy of the lengths (planning work,
    # outside the timed region)
    order = None if (args.no_order or not S) else pkv.longest_first(b.lens_dec)

    def do_decode(rep):
        pkv.paged_attention_decode(rep["q"], rep["kc"], rep["vc"], tab, lens,
                                   max_seq_len=max_len, scale=b.scale, out=rep["out"],
                                   workspace=rep["ws"], partition_size=args.partition_size,
                                   seq_order=order)

    def do_prefill(rep):
        pkv.paged_attention_prefill(rep["qp"], cu, rep["kc"], rep["vc"], tabp, lensp,
                                    max_q_len=max_q, max_seq_len=max_len_pf, scale=b.scale,
                                    out=rep["outp"], workspace=ws_pf)

    def step(rep):
        do_append(rep)
        if C:
            do_prefill(rep)
        if S:
            do_decode(rep)

    # warmup (eager), then capture one graph per replica
    for i in range(args.warmup):
        step(reps[i % R])
    torch.cuda.synchronize()
    graphs = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for rep in reps:
                step(rep)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for rep in reps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(rep)
            graphs.append(g)
        rounds = torch.cuda.CUDAGraph()   # R steps, one per replica
        with torch.cuda.graph(rounds):
            for rep in reps:
                step(rep)
        for g in graphs:   # replays double as extra warmup
            g.replay()
        rounds.replay()
        torch.cuda.synchronize()

    # timed region: exactly K steps
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    if graphs is not None:
        for _ in range(K // R):
            rounds.replay()
        for i in range(K // R * R, K):
            graphs[i % R].replay()
    else:
        for i in range(K):
            step(reps[i % R])
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = gpu_ms / K
    log(f"{name}: {K} steps: {gpu_ms:.3f} ms GPU, {wall_ms:.3f} ms wall")

    # the spread of whole steps: batches of back-to-back steps through the same
    # graphs (or eager steps), per-step time = batch time / steps per batch
    if graphs is not None:
        n_rounds = max(1, TIMING_CALLS // R)
        sst = launch_stats(lambda i: rounds.replay(), per_batch=n_rounds)
        steps_per_call = R
    else:
        sst = launch_stats(lambda i: step(reps[i % R]))
        steps_per_call = 1
    step_spread = {f"step_{k}": round(sst[k] / steps_per_call, 3)
                   for k in ("us_median", "us_p10", "us_p90")}

    # launch durations, independent of K (GPU kept ahead of the host)
    def timed(fn):
        return launch_stats(lambda i: fn(reps[i % R]))

    res = {}
    if S:
        res["decode"] = timed(do_decode)
    res["append"] = timed(do_append)
    if C:
        res["prefill"] = timed(do_prefill)

    step_s = ms_per_step / 1e3
    value = kv_bytes / step_s / 1e9 if S else 0.0
    rec = {
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_per_step, 6),
        "config": {
            "workload": name, "description": spec.description,
            "num_seqs": S, "prefill_chunks": C, "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
            "block_size": spec.block_size, "seq_lens_total": int(b.lens_dec.sum()) if S else 0,
            "max_seq_len": max_len, "partition_size": part, "replicas": R,
            "graph": graphs is not None,
            "dispatch_order": "batch" if order is None else "longest_first",
            "steps_per_graph": R if graphs is not None else 0,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round((S + C) / step_s, 1),
        "kv_bytes_per_step": kv_bytes,
        "kv_bytes_logical": kvb["logical"],
        "wall_ms_per_step": round(wall_ms / K, 6),
        **step_spread,
        "append_us_median": res["append"]["us_median"],
    }
    if S:
        st = res["decode"]
        achieved = decode_alg_bytes / (st["us_median"] * 1e-6) / 1e9
        rec["roofline"] = {
            "kernel": "paged_attention_decode (partition kernel + merge kernel when split)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(name),
            "alg_bytes_per_launch": decode_alg_bytes,
            **st,
        }
    if C:
        st = res["prefill"]
        tf = pf_flops / (st["us_median"] * 1e-6) / 1e12
        rec["prefill"] = {"flops": pf_flops, "tflops": round(tf, 1),
                          "frac_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                          "tokens_per_s": round(int(b.new_k.shape[0]) / step_s, 1), **st}
    del reps, graphs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_seconds:
        rec["cpu_baseline"] = cpu_baseline(b, kv_bytes, cpu_seconds)
    return rec


def main():
    args = parse()
    if args.stamp_source:
        stamp_source(args.stamp_source)
        return
    if args.summarize_pmc:
        summarize_pmc(args.workload or HEADLINE, *args.summarize_pmc)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_407_amd as pkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration()
        return
    pkv.load_library()
    log("library", pkv.LIB_PATH, "device", torch.cuda.get_device_name(dev))
    headline = args.workload or HEADLINE
    if args.block_size_sweep:
        block_size_sweep(args, dev, args.workload or "llama_decode")
        return
    if args.prefill_sweep:
        prefill_sweep(args, dev)
        return
    if args.swap_bench:
        swap_bench(args, dev, args.workload or "llama_decode")
        return
    if args.serve:
        serve_bench(args, dev, args.workload or "llama_decode")
        return

    if args.per_config is not None:
        extra = [w for w in args.per_config.split(",") if w]
    else:
        extra = [] if args.workload else list(PER_CONFIG)
    cpu = None if args.no_cpu_baseline else args.cpu_seconds
    rec = measure(headline, args, dev, cpu)
    line = {
        "metric": METRIC,
        "value": rec.pop("value"),
        "unit": rec.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic",
        "config": rec.pop("config"),
    }
    line.update(rec)
    if extra:
        line["per_config"] = {}
        for name in extra:
            line["per_config"][name] = measure(name, args, dev, cpu and cpu / 3)
    recs = [line, *line.get("per_config", {}).values()]
    same = [r["roofline"]["alg_bytes_per_launch"] // 16 * 16 for r in recs if "roofline" in r]
    sr, sr_sized = stream_read_reference(dev, same)
    line["stream_read"] = sr
    for r in recs:
        if "roofline" in r:
            rl = r["roofline"]
            rl["frac_of_stream_read"] = round(rl["achieved"] / sr["GBps"], 4)
            ref = sr_sized.get(rl["alg_bytes_per_launch"] // 16 * 16)
            if ref:
                rl["stream_read_same_bytes"] = ref
                rl["frac_of_stream_read_same_bytes"] = round(rl["achieved"] / ref["GBps"], 4)
    mr = mfma_reference(dev)
    line["mfma_reference"] = mr
    for r in [line, *line.get("per_config", {}).values()]:
        if "prefill" in r:
            r["prefill"]["frac_of_mfma_reference"] = round(
                r["prefill"]["tflops"] / mr["f16_16x16x32"]["TFLOPs"], 4)
    print(json.dumps(line), flush=True)


SWEEP_BLOCK_SIZES = (1, 8, 16, 32)


def block_size_sweep(args, dev, workload):
    """Decode of one batch at several block sizes: the same seeded lengths,
    queries and KV contents, the pool holding the same number of tokens
    (num_blocks * block_size fixed), each block table as wide as the longest
    sequence needs.  Cold caches as in the main run (replicas), per-call
    launch durations (launch_stats) with the GPU kept ahead of the host."""
    import dataclasses
    import torch
    import paged_kv_cache_407_amd as pkv
    base = W.SPECS[workload]
    if base.shared_prefix or base.prefill_chunks:
        raise SystemExit("the sweep takes a decode-only workload without sharing")
    tokens = base.num_blocks * base.block_size
    for bs in SWEEP_BLOCK_SIZES:
        spec = dataclasses.replace(base, name=f"{base.name}_bs{bs}", block_size=bs,
                                   num_blocks=tokens // bs, max_blocks_per_seq=0)
        b = W.make_batch(spec)
        S, Hq, D = b.q_dec.shape
        max_len = int(b.lens_dec.max())
        kv_bytes = W.decode_kv_bytes(b)["logical"]
        alg = kv_bytes + b.q_dec.nbytes + S * Hq * D * 4
        part = pkv.decode_partition_size(S, Hq, spec.num_kv_heads, D, bs, max_len,
                                         args.partition_size)
        wsb = pkv.decode_workspace_size(S, Hq, spec.num_kv_heads, D, bs, max_len,
                                        args.partition_size)
        R = max(1, min(16, math.ceil(2.0e9 / kv_bytes), int(64e9 // b.nbytes_pool())))

        def to_dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.float16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.float16)
            return torch.from_numpy(a).to(dev)
        nk, nv, slots = to_dev(b.new_k), to_dev(b.new_v), to_dev(b.slot_mapping)
        tab, lens, q = to_dev(b.tables_dec), to_dev(b.lens_dec), to_dev(b.q_dec)
        order = None if args.no_order else pkv.longest_first(b.lens_dec)
        reps = []
        for r in range(R):
            kc, vc = to_dev(b.k_cache), to_dev(b.v_cache)
            pkv.kv_append(nk, nv, kc, vc, slots)
            reps.append((kc, vc, torch.empty((S, Hq, D), dtype=torch.float32, device=dev),
                         torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None))

        def call(rep):
            kc, vc, out, ws = rep
            pkv.paged_attention_decode(q, kc, vc, tab, lens, max_seq_len=max_len,
                                       scale=b.scale, out=out, workspace=ws,
                                       partition_size=args.partition_size,
                                       seq_order=order)
        for i in range(args.warmup):
            call(reps[i % R])
        st = launch_stats(lambda i: call(reps[i % R]))
        mean = st["us_median"]
        gbs = alg / (mean * 1e-6) / 1e9
        log(f"block size {bs:2d}: decode {mean:8.2f} us, {gbs:7.1f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:5.1f} % of HBM peak), partition {part}, "
            f"table width {b.tables_dec.shape[1]}, replicas {R}")
        print(json.dumps({
            "metric": "paged decode GB/s by block size", "workload": workload,
            "block_size": bs, "num_blocks": spec.num_blocks,
            "table_entries": int(sum(W.cdiv(int(L), bs) for L in b.lens_dec)),
            "partition_size": part, **st,
            "alg_bytes": alg, "GBps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "replicas": R}),
            flush=True)
        del reps
        torch.cuda.empty_cache()


# (label, chunks, new tokens per chunk, prefix lo, prefix hi) at the 32 x 128
# MHA shape with block size 16
PREFILL_SWEEP = [
    ("1 chunk x 512 on a 3584-token prefix", 1, 512, 3584, 3584),
    ("1 chunk x 512 on a 1536-token prefix", 1, 512, 1536, 1536),
    ("2 chunks x 256 on prefixes U[1024,2048]", 2, 256, 1024, 2048),
    ("1 chunk x 2048 on an empty prefix", 1, 2048, 0, 0),
    ("4 chunks x 512 on prefixes U[0,512]", 4, 512, 0, 512),
]


def prefill_sweep(args, dev):
    """Prefill alone on batches whose query tiles are few (one or two
    chunks on long prefixes: the library cuts their key ranges across
    workgroups and merges the parts) and on the mixed step's 4 chunks
    (not split).  Launch durations as launch_stats measures them, caches cold
    across replicas."""
    import torch
    import paged_kv_cache_407_amd as pkv
    base = W.SPECS["mixed"]
    for i, (label, C, clen, plo, phi) in enumerate(PREFILL_SWEEP):
        spec = W.Spec(name=f"prefill_sweep_{i}", num_q_heads=base.num_q_heads,
                      num_kv_heads=base.num_kv_heads, head_dim=base.head_dim,
                      block_size=base.block_size,
                      num_blocks=C * W.cdiv(clen + phi, base.block_size) + 8,
                      seed=W.SEED_BASE + 20 + i, prefill_chunks=C, prefill_chunk_len=clen,
                      prefill_prefix_lo=plo, prefill_prefix_hi=phi)
        b = W.make_batch(spec)
        T, Hq, D = b.q_pf.shape
        max_q = int(np.diff(b.cu_q_lens).max())
        max_len = int(b.lens_pf.max())
        flops = W.prefill_flops(b)
        wsb = pkv.prefill_workspace_size(C, T, max_q, Hq, D, max_len)
        R = max(1, min(8, int(16e9 // b.nbytes_pool())))

        def to_dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.float16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.float16)
            return torch.from_numpy(a).to(dev)
        nk, nv, slots = to_dev(b.new_k), to_dev(b.new_v), to_dev(b.slot_mapping)
        q, cu = to_dev(b.q_pf), to_dev(b.cu_q_lens)
        tab, lens = to_dev(b.tables_pf), to_dev(b.lens_pf)
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
        reps = []
        for r in range(R):
            kc, vc = to_dev(b.k_cache), to_dev(b.v_cache)
            pkv.kv_append(nk, nv, kc, vc, slots)
            reps.append((kc, vc))

        def call(rep):
            pkv.paged_attention_prefill(q, cu, rep[0], rep[1], tab, lens, max_q_len=max_q,
                                        max_seq_len=max_len, scale=b.scale, out=out,
                                        workspace=ws)
        for j in range(args.warmup):
            call(reps[j % R])
        st = launch_stats(lambda j: call(reps[j % R]))
        mean = st["us_median"]
        tf = flops / (mean * 1e-6) / 1e12
        log(f"{label}: prefill {mean:8.2f} us, {tf:6.1f} TFLOP/s "
            f"({100 * tf / MFMA_F16_PEAK_TFLOPS:5.1f} % of fp16 MFMA peak), "
            f"{'split, workspace %.1f MiB' % (wsb / 2**20) if wsb else 'not split'}")
        print(json.dumps({
            "metric": "paged causal prefill TFLOP/s", "case": label, "chunks": C,
            "chunk_len": clen, "prefixes": (b.lens_pf - clen).tolist(),
            "num_q_heads": Hq, "num_kv_heads": spec.num_kv_heads, "head_dim": D,
            "block_size": spec.block_size, "flops": flops, **st,
            "tflops": round(tf, 1), "frac_mfma_f16_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "split": bool(wsb), "workspace_bytes": wsb, "replicas": R}),
            flush=True)
        del reps
        torch.cuda.empty_cache()


def swap_bench(args, dev, workload):
    """Swap-out (device pool -> pinned host pool) and swap-in (back) of
    ``--swap-blocks`` blocks scattered over the workload's device pool, to
    consecutive host blocks and back to other scattered device blocks: the
    kernel path (device id lists, one launch) and the DMA path (host id
    lists, hipMemcpyAsync per run).  Bytes = blocks x 2 (K, V) x Hkv x bs x
    D x 2 each way; the host link bounds both."""
    import torch
    import paged_kv_cache_407_amd as pkv
    spec = W.SPECS[workload]
    NB, Hkv, bs, D = spec.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim
    n = min(args.swap_blocks, NB)
    rng = np.random.default_rng(1)
    dk = torch.randn((NB, Hkv, bs, D), device=dev).half()
    dv = torch.randn((NB, Hkv, bs, D), device=dev).half()
    hk = torch.empty((n, Hkv, bs, D), dtype=torch.float16, pin_memory=True)
    hv = torch.empty((n, Hkv, bs, D), dtype=torch.float16, pin_memory=True)
    out_src = rng.permutation(NB)[:n].astype(np.int32)
    in_dst = rng.permutation(NB)[:n].astype(np.int32)
    host = np.arange(n, dtype=np.int32)
    ids = {k: torch.from_numpy(v).to(dev) for k, v in
           (("out_src", out_src), ("in_dst", in_dst), ("host", host))}
    nbytes = n * 2 * Hkv * bs * D * 2
    cases = [
        ("out", "kernel", lambda: pkv.copy_blocks(dk, dv, hk, hv, ids["out_src"], ids["host"])),
        ("in", "kernel", lambda: pkv.copy_blocks(hk, hv, dk, dv, ids["host"], ids["in_dst"])),
        ("out", "dma", lambda: pkv.copy_blocks_dma(dk, dv, hk, hv, out_src, host)),
        ("in", "dma", lambda: pkv.copy_blocks_dma(hk, hv, dk, dv, host, in_dst)),
    ]
    for direction, path, fn in cases:
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        reps = max(3, min(args.steps, 20))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        d = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e3
        gbs = nbytes / (d.mean() * 1e-6) / 1e9
        log(f"swap {direction:3s} {path:6s}: {n} blocks, {nbytes / 1e6:.1f} MB, "
            f"{d.mean():9.1f} us, {gbs:6.1f} GB/s")
        print(json.dumps({"metric": "KV block swap GB/s", "direction": direction,
                          "path": path, "workload": workload, "blocks": n,
                          "bytes": nbytes, "us_mean": round(float(d.mean()), 1),
                          "GBps": round(gbs, 2), "calls": reps}), flush=True)


def serve_bench(args, dev, workload):
    """Sustained multi-step continuous batching at the workload's attention
    shape: every request is queued at the start (prompt ~ U[64, 1024] tokens
    as in the pages' batch-32 comparison, generation ~ U[16, 256] tokens),
    and the native scheduler's plans drive kv_append, the prefill chunks and
    the decode rows until all have finished.  Query/key/value rows come from
    a resident random buffer (their values do not change the work).  Reports
    sequence-steps per second (prefill rows + decode rows per second of wall
    time, host scheduling included), tokens per second, and the share of the
    wall time the host spends planning (scheduler, staging buffer wait,
    plan copy enqueue)."""
    import torch
    import paged_kv_cache_407_amd as pkv
    from paged_kv_cache_407_amd.driver import StepDriver
    spec = W.SPECS[workload]
    NB, Hq, Hkv, D, bs = (spec.num_blocks, spec.num_q_heads, spec.num_kv_heads,
                          spec.head_dim, spec.block_size)
    B, T, max_len = args.serve_batch, args.serve_tokens, 1024 + 256
    rng = np.random.default_rng(11)
    n = args.serve_requests
    prompts = rng.integers(64, 1025, size=n)
    gens = rng.integers(16, 257, size=n)
    kc = torch.randn((NB, Hkv, bs, D), device=dev).half()
    vc = torch.randn((NB, Hkv, bs, D), device=dev).half()
    rows = T + B
    rk = torch.randn((rows, Hkv, D), device=dev).half()
    rv = torch.randn((rows, Hkv, D), device=dev).half()
    rq = torch.randn((rows, Hq, D), device=dev).half()
    scale = float(np.float32(1 / math.sqrt(D)))

    def rows_fn(plan):
        nt = plan["num_new_tokens"]
        return rk[:nt], rv[:nt], rq[:nt]

    def run(count, record):
        bm = pkv.BlockManager(NB - 1, bs)
        sch = pkv.Scheduler(bm, B, T, max_len)
        for i in range(count):
            sch.add_request(i, int(prompts[i]), int(gens[i]))
        drv = StepDriver(sch, kc, vc, Hq, scale, rows_fn, pad_block=NB - 1)
        st = dict(steps=0, rows=0, prefill_rows=0, decode_rows=0, prefill_tokens=0,
                  finished=0, preempted=0, host_s=0.0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while st["finished"] < count:
            h0 = time.perf_counter()
            plan, _, _ = drv.step()
            st["host_s"] += time.perf_counter() - h0
            st["steps"] += 1
            st["prefill_rows"] += len(plan["prefill_ids"])
            st["decode_rows"] += len(plan["decode_ids"])
            st["prefill_tokens"] += int(plan["cu_q_lens"][-1])
            st["finished"] += len(plan["finished"])
            st["preempted"] += len(plan["preempted"])
        torch.cuda.synchronize()
        st["wall_s"] = time.perf_counter() - t0
        st["plan_s"] = drv.plan_s
        drv.close()
        return st

    run(min(n, 2 * B), False)                         # warm-up (kernels, allocator)
    st = run(n, True)
    seq_steps = st["prefill_rows"] + st["decode_rows"]
    log(f"serve: {n} requests, {st['steps']} steps, {st['wall_s'] * 1e3:.1f} ms, "
        f"{seq_steps / st['wall_s']:.0f} seq-steps/s, {st['decode_rows'] / st['wall_s']:.0f} "
        f"decode tokens/s, {st['preempted']} preempted")
    print(json.dumps({
        "metric": "seq-steps/s (multi-step continuous batching)", "workload": workload,
        "value": round(seq_steps / st["wall_s"], 1), "unit": "seq-steps/s",
        "requests": n, "max_batch_size": B, "max_num_tokens": T, "steps": st["steps"],
        "wall_ms": round(st["wall_s"] * 1e3, 2),
        "ms_per_step": round(st["wall_s"] * 1e3 / st["steps"], 4),
        "decode_tokens_per_s": round(st["decode_rows"] / st["wall_s"], 1),
        "prefill_tokens_per_s": round(st["prefill_tokens"] / st["wall_s"], 1),
        "requests_per_s": round(n / st["wall_s"], 2),
        "host_share": round(st["host_s"] / st["wall_s"], 3),
        "plan_share": round(st["plan_s"] / st["wall_s"], 4),
        "preempted": st["preempted"], "prompt_tokens": int(prompts.sum()),
        "generated_tokens": int(gens.sum()),
        "config": {"num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "num_blocks": NB, "prompt": "U[64,1024]", "generate": "U[16,256]"}}),
        flush=True)


def cpu_baseline(b: W.Batch, kv_bytes: int, budget_s: float) -> dict:
    """The CPU oracle's kv append + decode (+ prefill) of this batch on the
    host cores.  The oracle writes the append into pools it owns, so the
    batch's pools are copied once before any clock starts; every run then
    appends the step's rows in place (the same rows to the same slots, so
    runs are identical) and attends over a seeded sample of (row, head)
    items.  The sample is sized from a short calibration run so that one run
    takes about budget_s / 3; the attention time is scaled to the whole batch
    by the sampled share of the attention work (keys attended, summed over
    the items).  Median of 3 runs with all host threads; one run on one
    thread with a third of the budget."""
    import oracle
    orc = oracle.get()
    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    S, Hq = b.num_dec, b.spec.num_q_heads
    T = b.q_pf.shape[0] if b.num_pf else 0
    # work items: (kind, row id, keys attended); kind 0 = decode, 1 = prefill
    kinds, ids, keys = [], [], []
    if S:
        r = np.arange(S * Hq, dtype=np.int64)
        kinds.append(np.zeros(r.size, np.int8))
        ids.append(r)
        keys.append(np.repeat(b.lens_dec.astype(np.int64), Hq))
    if T:
        per_tok = np.empty(T, np.int64)
        for c in range(b.num_pf):
            lo, hi = int(b.cu_q_lens[c]), int(b.cu_q_lens[c + 1])
            P = int(b.lens_pf[c]) - (hi - lo)
            per_tok[lo:hi] = P + 1 + np.arange(hi - lo)
        r = np.arange(T * Hq, dtype=np.int64)
        kinds.append(np.ones(r.size, np.int8))
        ids.append(r)
        keys.append(np.repeat(per_tok, Hq))
    kinds, ids, keys = np.concatenate(kinds), np.concatenate(ids), np.concatenate(keys)
    total_keys = int(keys.sum())
    perm = np.random.default_rng(0).permutation(ids.size)
    csum = np.cumsum(keys[perm])

    t0 = time.perf_counter()
    kc, vc = np.array(b.k_cache, copy=True), np.array(b.v_cache, copy=True)
    log(f"cpu baseline: pool copy {time.perf_counter() - t0:.1f}s (not timed)")

    def pick(n_items):
        sel = np.sort(perm[:n_items])
        dec = ids[sel][kinds[sel] == 0]
        pf = ids[sel][kinds[sel] == 1]
        return dec, pf, float(keys[sel].sum()) / total_keys

    def run(dec_rows, pf_rows, frac):
        t0 = time.perf_counter()
        orc.kv_append_inplace(b.new_k, b.new_v, kc, vc, b.slot_mapping)
        t_app = time.perf_counter() - t0
        t0 = time.perf_counter()
        if dec_rows.size:
            orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale, rows=dec_rows)
        if pf_rows.size:
            orc.prefill(b.q_pf, b.cu_q_lens, kc, vc, b.tables_pf, b.lens_pf, b.scale,
                        rows=pf_rows)
        return t_app + (time.perf_counter() - t0) / frac

    def sized(threads, run_budget):
        """Items whose attention takes about run_budget seconds."""
        orc.set_threads(threads)
        n0 = min(ids.size, 4 * threads)
        d0, p0, f0 = pick(n0)
        t0 = time.perf_counter()
        if d0.size:
            orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale, rows=d0)
        if p0.size:
            orc.prefill(b.q_pf, b.cu_q_lens, kc, vc, b.tables_pf, b.lens_pf, b.scale, rows=p0)
        per_key = (time.perf_counter() - t0) / max(1.0, f0 * total_keys)
        want = run_budget / max(per_key, 1e-12)
        n = int(np.searchsorted(csum, want)) + 1
        return pick(max(n0, min(ids.size, n)))

    try:
        dec, pf, frac = sized(cores, budget_s / 3)
        steps = sorted(run(dec, pf, frac) for _ in range(3))
        step = steps[1]
        dec1, pf1, frac1 = sized(1, budget_s / 3)
        step1 = run(dec1, pf1, frac1)
    finally:
        orc.set_threads(0)
    what = "decode" + (" and prefill" if T else "")
    return {"value": round(kv_bytes / step / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"median of 3 runs; each run: the oracle's kv append of all "
                      f"{b.new_k.shape[0]} new rows (in place, pool copy made before "
                      f"timing) plus its {what} over {dec.size + pf.size} of {ids.size} "
                      f"(row, head) items = {frac:.2%} of the attention work (keys "
                      f"attended); attention time scaled to the whole batch",
            "step_s": round(step, 4), "step_s_runs": [round(x, 4) for x in steps],
            "cpu": _cpu_model(),
            "single_thread": {"value": round(kv_bytes / step1 / 1e9, 4), "cores": 1,
                              "step_s": round(step1, 4),
                              "sample": f"one run on one thread: kv append plus {what} over "
                                        f"{frac1:.2%} of the attention work, scaled"}}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
