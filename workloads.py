"""Seeded synthetic inputs for the paged-attention workloads.

This module only builds host (numpy) arrays: query rows, a K/V pool whose
physical blocks are handed out by a seeded random permutation, block tables,
sequence lengths, and the new K/V rows with their slot mapping.  It does no
attention arithmetic.  The HIP path and the CPU oracle both consume exactly
the arrays built here.

Pool layout is ``[num_blocks, num_kv_heads, block_size, head_dim]`` fp16; a
token at logical position ``t`` of a sequence whose block table row is
``table`` lives in physical block ``table[t // block_size]`` at offset
``t % block_size`` ("LLM 推理引擎 Continuous Batching 与 PagedAttention",
§3.2 BlockManager and §3.3 GPU kernel paged read).

Every slot that no live token occupies holds an fp16 NaN canary, and unused
block-table entries point at a reserved block that is NaN throughout, so any
read past a sequence's end surfaces as NaN in an output.

Draw order for one seed: lengths, block permutation, queries, then K/V
contents from one child stream per sequence (drawn in threads; each child is
independent, so the result does not depend on the thread count), then the
padding rows.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

FP16_NAN_BITS = 0x7E00
SEED_BASE = 4070


@dataclass(frozen=True)
class Spec:
    """Shape and length distribution of one workload."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seed: int
    # decode sequences
    decode_lens: tuple = ()            # fixed lengths, or empty
    decode_count: int = 0              # number of decode sequences when drawn
    decode_dist: str = ""              # "uniform" | "lognormal" | "const"
    decode_lo: int = 0
    decode_hi: int = 0
    decode_median: float = 0.0
    decode_sigma: float = 0.0
    # prefill chunks: chunk_len new tokens on a cached prefix ~ U{lo..hi}
    prefill_chunks: int = 0
    prefill_chunk_len: int = 0
    prefill_prefix_lo: int = 0
    prefill_prefix_hi: int = 0
    # tokens at the start of every decode sequence that map to one shared set
    # of physical blocks (system-prompt sharing)
    shared_prefix: int = 0
    max_blocks_per_seq: int = 0        # block-table width; 0 = derive
    description: str = ""


# The five workloads.  Lengths always count the token appended in this step.
SPECS = {
    "tiny": Spec(
        name="tiny", num_q_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
        num_blocks=64, seed=SEED_BASE + 1, decode_lens=(5, 16, 17, 40),
        description="tiny decode: 4 heads x 64, bs 16, 64-block pool, "
                    "lengths {5,16,17,40}"),
    "llama_decode": Spec(
        name="llama_decode", num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, num_blocks=4096, seed=SEED_BASE + 2, decode_count=32,
        decode_dist="uniform", decode_lo=64, decode_hi=1024,
        max_blocks_per_seq=64,
        description="Llama-2-7B-shaped single-layer decode: 32x128 MHA, bs 16, "
                    "batch 32, L~U[64,1024], 4096-block pool"),
    "mixed": Spec(
        name="mixed", num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, num_blocks=8192, seed=SEED_BASE + 3, decode_count=60,
        decode_dist="uniform", decode_lo=64, decode_hi=2048,
        prefill_chunks=4, prefill_chunk_len=512, prefill_prefix_lo=0,
        prefill_prefix_hi=512, max_blocks_per_seq=128,
        description="mixed step: 4 prefill chunks x 512 on prefixes U[0,512] "
                    "+ 60 decode sequences L~U[64,2048], 32x128, bs 16"),
    "long": Spec(
        name="long", num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=16, num_blocks=32768, seed=SEED_BASE + 4, decode_count=8,
        decode_dist="const", decode_lo=32768, decode_hi=32768,
        max_blocks_per_seq=2048,
        description="long-context decode: 8 sequences x 32768 tokens, 32x128, "
                    "bs 16, 32768-block pool"),
    "gqa_shared": Spec(
        name="gqa_shared", num_q_heads=64, num_kv_heads=8, head_dim=128,
        block_size=32, num_blocks=16384, seed=SEED_BASE + 5, decode_count=256,
        decode_dist="lognormal", decode_lo=256, decode_hi=4096,
        decode_median=1024.0, decode_sigma=math.log(4.0) / 2.0,
        shared_prefix=512, max_blocks_per_seq=128,
        description="high-concurrency GQA decode: 256 sequences, 64 q / 8 kv "
                    "heads x 128, bs 32, lognormal L (median 1024, clip "
                    "[256,4096]), 512-token prefix shared by all"),
    # Two more grouped-query shapes, beside the five above: 4 and 16 query
    # heads per KV head (the group sizes of 32/8- and 128/8-head models),
    # measured like the others but not part of the contract's five.
    "gqa4": Spec(
        name="gqa4", num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, num_blocks=64 * 192 + 64, seed=SEED_BASE + 6, decode_count=64,
        decode_dist="uniform", decode_lo=1024, decode_hi=3072, max_blocks_per_seq=192,
        description="grouped-query decode, 4 query heads per KV head: 64 sequences, "
                    "32 q / 8 kv heads x 128, bs 16, L~U[1024,3072]"),
    "gqa16": Spec(
        name="gqa16", num_q_heads=128, num_kv_heads=8, head_dim=128,
        block_size=16, num_blocks=64 * 192 + 64, seed=SEED_BASE + 7, decode_count=64,
        decode_dist="uniform", decode_lo=1024, decode_hi=3072, max_blocks_per_seq=192,
        description="grouped-query decode, 16 query heads per KV head: 64 sequences, "
                    "128 q / 8 kv heads x 128, bs 16, L~U[1024,3072]"),
}


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: int = 2) -> int:
    """K plus V bytes one token occupies: 2 x layers x heads x head_dim x bytes
    ("LLM 推理引擎 …", §1.2 KV Cache 的本质)."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Batch:
    spec: Spec
    scale: float
    k_cache: np.ndarray          # [NB, Hkv, bs, D] fp16, before the append
    v_cache: np.ndarray
    new_k: np.ndarray            # [T, Hkv, D] fp16
    new_v: np.ndarray
    slot_mapping: np.ndarray     # [T] int32, -1 = padding row
    canary_block: int
    max_blocks_per_seq: int
    # decode part (None when absent)
    q_dec: np.ndarray | None = None          # [S, Hq, D] fp16
    tables_dec: np.ndarray | None = None     # [S, MB] int32
    lens_dec: np.ndarray | None = None       # [S] int32
    # prefill part (None when absent)
    q_pf: np.ndarray | None = None           # [sum C, Hq, D] fp16
    cu_q_lens: np.ndarray | None = None      # [C+1] int32
    tables_pf: np.ndarray | None = None      # [C, MB] int32
    lens_pf: np.ndarray | None = None        # [C] int32 (prefix + chunk)
    # logical-order contents per sequence, decode sequences first then
    # prefill chunks: list of (K [L, Hkv, D], V [L, Hkv, D]); only when kept
    dense: list | None = None
    extra: dict = field(default_factory=dict)

    @property
    def num_dec(self) -> int:
        return 0 if self.lens_dec is None else int(self.lens_dec.shape[0])

    @property
    def num_pf(self) -> int:
        return 0 if self.lens_pf is None else int(self.lens_pf.shape[0])

    def nbytes_pool(self) -> int:
        return self.k_cache.nbytes + self.v_cache.nbytes


def _draw_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    if spec.decode_lens:
        return np.asarray(spec.decode_lens, dtype=np.int64)
    n = spec.decode_count
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    if spec.decode_dist == "uniform":
        return rng.integers(spec.decode_lo, spec.decode_hi, size=n,
                            endpoint=True)
    if spec.decode_dist == "const":
        return np.full(n, spec.decode_lo, dtype=np.int64)
    if spec.decode_dist == "lognormal":
        z = rng.standard_normal(n)
        raw = np.rint(np.exp(math.log(spec.decode_median) + spec.decode_sigma * z))
        return np.clip(raw, spec.decode_lo, spec.decode_hi).astype(np.int64)
    raise ValueError(spec.decode_dist)


def _normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def make_batch(spec: Spec | str, *, seed: int | None = None, pad_rows: int = 0,
               keep_dense: bool = False, threads: int | None = None,
               lens_override: dict | None = None) -> Batch:
    """Build one seeded batch of ``spec``.

    ``pad_rows`` adds that many extra rows with slot -1 (they must be
    skipped).  ``keep_dense`` keeps each sequence's logical-order K/V.
    ``lens_override`` may replace the drawn lengths: ``{"decode": [...],
    "prefix": [...]}`` (used by edge-case tests).
    """
    if isinstance(spec, str):
        spec = SPECS[spec]
    seed = spec.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, bs, NB = (spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                          spec.block_size, spec.num_blocks)

    # 1. lengths
    dec_lens = _draw_lengths(spec, rng)
    pf_prefix = (rng.integers(spec.prefill_prefix_lo, spec.prefill_prefix_hi,
                              size=spec.prefill_chunks, endpoint=True)
                 if spec.prefill_chunks else np.zeros(0, dtype=np.int64))
    if lens_override:
        if "decode" in lens_override:
            dec_lens = np.asarray(lens_override["decode"], dtype=np.int64)
        if "prefix" in lens_override:
            pf_prefix = np.asarray(lens_override["prefix"], dtype=np.int64)
    C = int(pf_prefix.shape[0])
    clen = spec.prefill_chunk_len
    pf_lens = pf_prefix + clen
    S = int(dec_lens.shape[0])

    # Sequence records in allocation order: prefill chunks, then decode.
    # (kind, index, L, new_start, shared_tokens)
    seqs = []
    for c in range(C):
        seqs.append(("pf", c, int(pf_lens[c]), int(pf_prefix[c]), 0))
    for s in range(S):
        L = int(dec_lens[s])
        shared = 0
        if spec.shared_prefix:
            # Full blocks of the shared prefix that do not hold this step's
            # new token stay shared; the block that receives the new token is
            # a private copy (copy-on-write).
            shared = min(spec.shared_prefix // bs, (L - 1) // bs) * bs
        seqs.append(("dec", s, L, L - 1, shared))

    max_len = max([r[2] for r in seqs], default=1)
    MB = spec.max_blocks_per_seq or cdiv(max_len, bs)
    if cdiv(max_len, bs) > MB:
        raise ValueError(f"{spec.name}: length {max_len} exceeds {MB} blocks")

    # 2. physical block assignment (block NB-1 is the all-NaN canary)
    canary = NB - 1
    perm = rng.permutation(NB - 1).astype(np.int64)
    cursor = 0
    shared_blocks = np.zeros(0, dtype=np.int64)
    if spec.shared_prefix:
        n_sh = spec.shared_prefix // bs
        shared_blocks = perm[:n_sh]
        cursor = n_sh
    tables = []
    for kind, idx, L, new_start, shared in seqs:
        nblk = cdiv(L, bs)
        n_sh = shared // bs
        own = nblk - n_sh
        if cursor + own > NB - 1:
            raise ValueError(f"{spec.name}: pool of {NB} blocks exhausted")
        row = np.full(MB, canary, dtype=np.int64)
        row[:n_sh] = shared_blocks[:n_sh]
        row[n_sh:nblk] = perm[cursor:cursor + own]
        cursor += own
        tables.append(row)

    # 3. queries
    q_pf = _normal_f16(rng, (C * clen, Hq, D)) if C else None
    q_dec = _normal_f16(rng, (S, Hq, D)) if S else None

    # 4. contents, one child stream per sequence (+1 for the shared prefix)
    kids = np.random.SeedSequence(seed).spawn(len(seqs) + 1)
    k_cache = np.full((NB, Hkv, bs, D), np.uint16(FP16_NAN_BITS),
                      dtype=np.uint16).view(np.float16)
    v_cache = np.full((NB, Hkv, bs, D), np.uint16(FP16_NAN_BITS),
                      dtype=np.uint16).view(np.float16)
    shared_k = shared_v = None
    if spec.shared_prefix:
        g = np.random.default_rng(kids[-1])
        shared_k = _normal_f16(g, (spec.shared_prefix, Hkv, D))
        shared_v = _normal_f16(g, (spec.shared_prefix, Hkv, D))
        n_sh = spec.shared_prefix // bs
        k_cache[shared_blocks] = shared_k.reshape(n_sh, bs, Hkv, D).transpose(0, 2, 1, 3)
        v_cache[shared_blocks] = shared_v.reshape(n_sh, bs, Hkv, D).transpose(0, 2, 1, 3)

    new_rows = [None] * len(seqs)
    dense = [None] * len(seqs) if keep_dense else None

    def fill(i):
        kind, idx, L, new_start, shared = seqs[i]
        g = np.random.default_rng(kids[i])
        # tokens before `priv` come from the shared prefix content
        priv = min(spec.shared_prefix, L - 1) if spec.shared_prefix else 0
        kp = _normal_f16(g, (L - priv, Hkv, D))
        vp = _normal_f16(g, (L - priv, Hkv, D))
        if priv:
            kd = np.concatenate([shared_k[:priv], kp])
            vd = np.concatenate([shared_v[:priv], vp])
        else:
            kd, vd = kp, vp
        nblk = cdiv(L, bs)
        n_sh = shared // bs
        row = tables[i]
        # stored tokens [0, new_start); the rest of the last block stays NaN
        kb = np.full((nblk * bs, Hkv, D), np.nan, dtype=np.float16)
        vb = np.full((nblk * bs, Hkv, D), np.nan, dtype=np.float16)
        kb[:new_start] = kd[:new_start]
        vb[:new_start] = vd[:new_start]
        kb = kb.reshape(nblk, bs, Hkv, D).transpose(0, 2, 1, 3)
        vb = vb.reshape(nblk, bs, Hkv, D).transpose(0, 2, 1, 3)
        k_cache[row[n_sh:nblk]] = kb[n_sh:]
        v_cache[row[n_sh:nblk]] = vb[n_sh:]
        pos = np.arange(new_start, L)
        slots = row[pos // bs] * bs + pos % bs
        new_rows[i] = (kd[new_start:L].copy(), vd[new_start:L].copy(), slots)
        if dense is not None:
            dense[i] = (kd, vd)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads > 1 and len(seqs) > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(len(seqs))))
    else:
        for i in range(len(seqs)):
            fill(i)

    new_k = np.concatenate([r[0] for r in new_rows]) if seqs else np.zeros((0, Hkv, D), np.float16)
    new_v = np.concatenate([r[1] for r in new_rows]) if seqs else np.zeros((0, Hkv, D), np.float16)
    slots = np.concatenate([r[2] for r in new_rows]).astype(np.int32) if seqs else np.zeros(0, np.int32)

    # 5. padding rows (slot -1): random data that must never land in the pool
    if pad_rows:
        at = np.sort(rng.choice(new_k.shape[0] + pad_rows, size=pad_rows, replace=False))
        keep = np.ones(new_k.shape[0] + pad_rows, dtype=bool)
        keep[at] = False
        nk = np.empty((keep.size, Hkv, D), np.float16)
        nv = np.empty((keep.size, Hkv, D), np.float16)
        ns = np.full(keep.size, -1, np.int32)
        nk[keep], nv[keep], ns[keep] = new_k, new_v, slots
        nk[~keep] = _normal_f16(rng, (pad_rows, Hkv, D))
        nv[~keep] = _normal_f16(rng, (pad_rows, Hkv, D))
        new_k, new_v, slots = nk, nv, ns

    tab = np.stack(tables).astype(np.int32) if seqs else np.zeros((0, MB), np.int32)
    b = Batch(spec=spec, scale=float(np.float32(1.0 / math.sqrt(D))),
              k_cache=k_cache, v_cache=v_cache, new_k=new_k, new_v=new_v,
              slot_mapping=slots, canary_block=canary, max_blocks_per_seq=MB)
    if C:
        b.q_pf = q_pf
        b.cu_q_lens = (np.arange(C + 1) * clen).astype(np.int32)
        b.tables_pf = np.ascontiguousarray(tab[:C])
        b.lens_pf = pf_lens.astype(np.int32)
    if S:
        b.q_dec = q_dec
        b.tables_dec = np.ascontiguousarray(tab[C:])
        b.lens_dec = dec_lens.astype(np.int32)
    if dense is not None:
        # decode sequences first, then prefill chunks
        b.dense = dense[C:] + dense[:C]
    b.extra["shared_blocks"] = shared_blocks
    return b


def kv_token_bytes(b: Batch) -> int:
    """K+V bytes of one token of one layer in this batch's pool."""
    return kv_bytes_per_token(1, b.spec.num_kv_heads, b.spec.head_dim)


def decode_kv_bytes(b: Batch) -> dict:
    """KV bytes the decode part must read: ``logical`` counts every valid
    token of every sequence, ``unique`` counts each physical (block, offset)
    once, so blocks shared by several sequences are counted once."""
    if b.lens_dec is None:
        return {"logical": 0, "unique": 0}
    per = kv_token_bytes(b)
    bs = b.spec.block_size
    logical = int(b.lens_dec.astype(np.int64).sum()) * per
    fill = {}
    for s in range(b.num_dec):
        L = int(b.lens_dec[s])
        for j in range(cdiv(L, bs)):
            p = int(b.tables_dec[s, j])
            fill[p] = max(fill.get(p, 0), min(bs, L - j * bs))
    unique = sum(fill.values()) * per
    return {"logical": logical, "unique": unique}


def prefill_flops(b: Batch) -> int:
    """Multiply-add work (x2) of the causal prefill chunks: every query row j
    of chunk c scores and weights ``prefix_c + j + 1`` keys, QK^T and PV."""
    if b.lens_pf is None:
        return 0
    D, Hq = b.spec.head_dim, b.spec.num_q_heads
    tot = 0
    for c in range(b.num_pf):
        C = int(b.cu_q_lens[c + 1] - b.cu_q_lens[c])
        P = int(b.lens_pf[c]) - C
        keys = C * P + C * (C + 1) // 2
        tot += 4 * D * Hq * keys
    return tot
