"""Helpers for the GPU parity tests: move a generated batch to the device and
run the library's entry points on it."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_cache_407_amd as pkv
import workloads as W

DEV = "cuda:0"


def say(*a):
    print("[gpu]", *a, file=sys.stderr, flush=True)


def to_dev(a: np.ndarray):
    if a.dtype == np.float16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.float16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float16:
        return t.view(torch.int16).cpu().numpy().view(np.float16)
    return t.cpu().numpy()


class DevBatch:
    """Device copies of a generated batch (pool before the append)."""

    def __init__(self, b: W.Batch):
        self.b = b
        self.k_cache = to_dev(b.k_cache)
        self.v_cache = to_dev(b.v_cache)
        self.new_k = to_dev(b.new_k)
        self.new_v = to_dev(b.new_v)
        self.slots = to_dev(b.slot_mapping)
        if b.num_dec:
            self.q_dec = to_dev(b.q_dec)
            self.tables_dec = to_dev(b.tables_dec)
            self.lens_dec = to_dev(b.lens_dec)
            self.max_len_dec = int(b.lens_dec.max())
        if b.num_pf:
            self.q_pf = to_dev(b.q_pf)
            self.cu = to_dev(b.cu_q_lens)
            self.tables_pf = to_dev(b.tables_pf)
            self.lens_pf = to_dev(b.lens_pf)
            self.max_q = int(np.diff(b.cu_q_lens).max())

    def append(self):
        pkv.kv_append(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slots)

    def decode(self, partition_size=0, tables=None, lens=None, max_seq_len=None,
               k_cache=None, v_cache=None, seq_order=None):
        return pkv.paged_attention_decode(
            self.q_dec, self.k_cache if k_cache is None else k_cache,
            self.v_cache if v_cache is None else v_cache,
            self.tables_dec if tables is None else tables,
            self.lens_dec if lens is None else lens,
            max_seq_len=max_seq_len or self.max_len_dec, scale=self.b.scale,
            partition_size=partition_size, seq_order=seq_order)

    def prefill(self, tables=None, k_cache=None, v_cache=None):
        return pkv.paged_attention_prefill(
            self.q_pf, self.cu, self.k_cache if k_cache is None else k_cache,
            self.v_cache if v_cache is None else v_cache,
            self.tables_pf if tables is None else tables, self.lens_pf,
            max_q_len=self.max_q, max_seq_len=int(self.b.lens_pf.max()), scale=self.b.scale)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
