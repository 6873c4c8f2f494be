"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises
``AssertionError`` when the oracle disagrees with what it is pinned to:

* torch's scaled-dot-product attention in float64 over the logical-order K/V
  the input generator drew before it scattered them into blocks (a library
  routine for the plain definition of attention; for chunks on a prefix the
  library's own causal rule is applied to the whole sequence);
* closed forms (one token, a zero query, one dominant key);
* bitwise invariance under relabelling physical blocks and under replacing
  shared blocks with private copies;
* hand-derived fixtures under ``tests/golden`` from the pages' examples;
* numpy's binary16 decoding for every one of the 65,536 bit patterns.

The same functions run against copies of the oracle with planted mistakes
(``test_oracle_mutations.py``), which must each fail at least one pin.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import replace

import numpy as np
import torch
import torch.nn.functional as F

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- workloads
def small_specs():
    """Small decode / mixed specs spanning block sizes 1, 2, 16 and GQA."""
    base = dict(num_blocks=0, seed=0)
    out = []
    for i, (Hq, Hkv, D, bs, lens) in enumerate([
        (2, 2, 8, 1, (1, 3, 7)),
        (4, 2, 8, 2, (1, 2, 5, 9)),
        (4, 1, 16, 16, (16, 17, 33, 40)),
        (8, 2, 64, 16, (5, 31, 32, 47)),
        (4, 4, 64, 16, (5, 16, 17, 40)),
    ]):
        nb = sum(W.cdiv(L, bs) for L in lens) + 7
        out.append(W.Spec(name=f"small{i}", num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=D, block_size=bs, num_blocks=nb,
                          seed=100 + i, decode_lens=lens))
    return out


def small_mixed_spec():
    return W.Spec(name="small_mixed", num_q_heads=4, num_kv_heads=2, head_dim=16,
                  block_size=4, num_blocks=128, seed=77, decode_count=3,
                  decode_dist="uniform", decode_lo=1, decode_hi=30,
                  prefill_chunks=3, prefill_chunk_len=9, prefill_prefix_lo=0,
                  prefill_prefix_hi=13)


def small_shared_spec():
    return W.Spec(name="small_shared", num_q_heads=8, num_kv_heads=2, head_dim=16,
                  block_size=4, num_blocks=256, seed=55, decode_count=9,
                  decode_dist="uniform", decode_lo=3, decode_hi=40,
                  shared_prefix=16)


# ---------------------------------------------------------------- references
def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.float64))


def sdpa(q, k, v, scale, causal=False):
    """q [Lq, Hq, D], k/v [Lk, Hkv, D] -> [Lq, Hq, D] float64."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = _t(q).permute(1, 0, 2).unsqueeze(0)
    kt = _t(k).permute(1, 0, 2).unsqueeze(0)
    vt = _t(v).permute(1, 0, 2).unsqueeze(0)
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, is_causal=causal,
                                       enable_gqa=(Hq != Hkv))
    return o[0].permute(1, 0, 2).numpy()


def dense_decode_reference(b: W.Batch):
    out = np.empty((b.num_dec,) + b.q_dec.shape[1:], np.float64)
    for s in range(b.num_dec):
        k, v = b.dense[s]
        out[s] = sdpa(b.q_dec[s:s + 1], k, v, b.scale)[0]
    return out


def dense_prefill_reference(b: W.Batch):
    """Runs the library's causal attention over the whole sequence (queries
    before the chunk are filler) and keeps the chunk's rows."""
    out = np.empty(b.q_pf.shape, np.float64)
    for c in range(b.num_pf):
        k, v = b.dense[b.num_dec + c]
        L = k.shape[0]
        lo, hi = int(b.cu_q_lens[c]), int(b.cu_q_lens[c + 1])
        P = L - (hi - lo)
        qf = np.zeros((L,) + b.q_pf.shape[1:], np.float16)
        qf[P:] = b.q_pf[lo:hi]
        out[lo:hi] = sdpa(qf, k, v, b.scale, causal=True)[P:]
    return out


def appended(orc, b: W.Batch):
    return orc.kv_append(b.new_k, b.new_v, b.k_cache, b.v_cache, b.slot_mapping)


# ---------------------------------------------------------------------- pins
def pin_half_decoding(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(x)) for x in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "binary16 decoding differs"


def pin_dense_decode(orc, spec, tol=1e-12, **kw):
    b = W.make_batch(spec, keep_dense=True, pad_rows=2, **kw)
    kc, vc = appended(orc, b)
    got = orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale)
    ref = dense_decode_reference(b)
    err = float(np.max(np.abs(got - ref)))
    assert err <= tol, f"{spec.name}: decode vs dense attention {err:.3g}"
    return err


def pin_dense_prefill(orc, spec, tol=1e-12):
    b = W.make_batch(spec, keep_dense=True)
    kc, vc = appended(orc, b)
    got = orc.prefill(b.q_pf, b.cu_q_lens, kc, vc, b.tables_pf, b.lens_pf, b.scale)
    ref = dense_prefill_reference(b)
    err = float(np.max(np.abs(got - ref)))
    assert err <= tol, f"{spec.name}: prefill vs dense causal attention {err:.3g}"
    if b.num_dec:
        gd = orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale)
        rd = dense_decode_reference(b)
        e2 = float(np.max(np.abs(gd - rd)))
        assert e2 <= tol, f"{spec.name}: mixed-step decode {e2:.3g}"
    return err


def pin_dense_config(orc, name, n_rows=48, seed=0, tol=1e-12):
    """Dense equivalence at a benchmark workload's real shape and pool: the
    oracle, reading through the block tables of the full batch, against
    torch's float64 attention over the logical-order K/V the generator drew
    (for every sequence that owns a sampled row; causal over the whole
    sequence for prefill chunks).  A seeded sample of n_rows (row, head)
    pairs of the decode part and of the prefill part, first and last rows
    included.  The batch's own pools take the append in place."""
    b = W.make_batch(name, keep_dense=True)
    kc = np.array(b.k_cache, copy=True)
    vc = np.array(b.v_cache, copy=True)
    orc.kv_append_inplace(b.new_k, b.new_v, kc, vc, b.slot_mapping)
    rng = np.random.default_rng(seed)
    worst = 0.0

    def sample(n):
        r = rng.choice(n, size=min(n, n_rows - 2), replace=False)
        return np.unique(np.concatenate([[0, n - 1], r])).astype(np.int64)

    if b.num_dec:
        S, Hq, D = b.q_dec.shape
        rows = sample(S * Hq)
        got = orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale,
                         rows=rows).reshape(S * Hq, D)
        for s in np.unique(rows // Hq):
            k, v = b.dense[s]
            ref = sdpa(b.q_dec[s:s + 1], k, v, b.scale)[0]
            for r in rows[rows // Hq == s]:
                worst = max(worst, float(np.max(np.abs(got[r] - ref[r % Hq]))))
    if b.num_pf:
        T, Hq, D = b.q_pf.shape
        rows = sample(T * Hq)
        got = orc.prefill(b.q_pf, b.cu_q_lens, kc, vc, b.tables_pf, b.lens_pf, b.scale,
                          rows=rows).reshape(T * Hq, D)
        tok = rows // Hq
        for c in range(b.num_pf):
            lo, hi = int(b.cu_q_lens[c]), int(b.cu_q_lens[c + 1])
            mine = rows[(tok >= lo) & (tok < hi)]
            if mine.size == 0:
                continue
            k, v = b.dense[b.num_dec + c]
            L = k.shape[0]
            P = L - (hi - lo)
            qf = np.zeros((L,) + b.q_pf.shape[1:], np.float16)
            qf[P:] = b.q_pf[lo:hi]
            ref = sdpa(qf, k, v, b.scale, causal=True)[P:]
            for r in mine:
                worst = max(worst, float(np.max(np.abs(got[r] - ref[r // Hq - lo, r % Hq]))))
    assert worst <= tol, f"{name}: oracle vs dense attention {worst:.3g}"
    return worst


def _single_seq_pool(rng, L, Hkv, D, bs, k=None, v=None):
    nblk = W.cdiv(L, bs)
    NB = nblk + 2
    kc = np.full((NB, Hkv, bs, D), np.nan, np.float16)
    vc = np.full((NB, Hkv, bs, D), np.nan, np.float16)
    order = rng.permutation(NB - 1)[:nblk]
    k = rng.standard_normal((L, Hkv, D)).astype(np.float16) if k is None else k
    v = rng.standard_normal((L, Hkv, D)).astype(np.float16) if v is None else v
    for t in range(L):
        kc[order[t // bs], :, t % bs] = k[t]
        vc[order[t // bs], :, t % bs] = v[t]
    table = np.full((1, nblk + 1), NB - 1, np.int32)
    table[0, :nblk] = order
    return kc, vc, table, k, v


def pin_closed_forms(orc):
    rng = np.random.default_rng(9)
    Hkv, D, bs = 2, 16, 4
    # one token: the output is that token's value, exactly
    kc, vc, tab, k, v = _single_seq_pool(rng, 1, Hkv, D, bs)
    q = rng.standard_normal((1, 4, D)).astype(np.float16)
    o = orc.decode(q, kc, vc, tab, np.array([1], np.int32), 0.25)
    for h in range(4):
        assert np.array_equal(o[0, h], v[0, h // 2].astype(np.float64)), "L=1"
    # zero query: uniform weights, the output is the mean of the values
    L = 23
    kc, vc, tab, k, v = _single_seq_pool(rng, L, Hkv, D, bs)
    q = np.zeros((1, 4, D), np.float16)
    o = orc.decode(q, kc, vc, tab, np.array([L], np.int32), 0.25)
    mean = v.astype(np.float64).mean(axis=0)
    for h in range(4):
        assert np.max(np.abs(o[0, h] - mean[h // 2])) < 1e-12, "q=0 mean"
    # all keys equal: uniform weights as well
    kk = np.repeat(rng.standard_normal((1, Hkv, D)).astype(np.float16), L, axis=0)
    kc, vc, tab, k, v = _single_seq_pool(rng, L, Hkv, D, bs, k=kk)
    q = rng.standard_normal((1, 4, D)).astype(np.float16)
    o = orc.decode(q, kc, vc, tab, np.array([L], np.int32), 0.25)
    mean = v.astype(np.float64).mean(axis=0)
    for h in range(4):
        assert np.max(np.abs(o[0, h] - mean[h // 2])) < 1e-12, "equal keys"
    # one dominant key at position 13 (score gap > 700): output = its value
    kk = np.zeros((L, Hkv, D), np.float16)
    kk[13] = 8.0
    kc, vc, tab, k, v = _single_seq_pool(rng, L, Hkv, D, bs, k=kk)
    q = np.full((1, 4, D), 8.0, np.float16)
    o = orc.decode(q, kc, vc, tab, np.array([L], np.int32), 1.0)
    for h in range(4):
        assert np.max(np.abs(o[0, h] - v[13, h // 2])) < 1e-12, "dominant key"
    # dominant key in a prefill row: row j sees it only once 13 <= prefix + j
    P, C = 10, 8
    qp = np.full((C, 4, D), 8.0, np.float16)
    cu = np.array([0, C], np.int32)
    o = orc.prefill(qp, cu, kc, vc, tab, np.array([P + C], np.int32), 1.0)
    for j in range(C):
        for h in range(4):
            if P + j >= 13:
                assert np.max(np.abs(o[j, h] - v[13, h // 2])) < 1e-12, "causal hit"
            else:
                mean = v[:P + j + 1, h // 2].astype(np.float64).mean(axis=0)
                assert np.max(np.abs(o[j, h] - mean)) < 1e-12, "causal mean"


def relabel_blocks(rng, b: W.Batch, kc, vc):
    """Moves every physical block p to pi(p) and rewrites the tables."""
    NB = kc.shape[0]
    pi = rng.permutation(NB)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    out = {}
    for name in ("tables_dec", "tables_pf"):
        t = getattr(b, name)
        out[name] = None if t is None else pi[t].astype(np.int32)
    return kc2, vc2, out


def pin_permutation_invariance(orc, spec):
    b = W.make_batch(spec)
    kc, vc = appended(orc, b)
    kc2, vc2, t2 = relabel_blocks(np.random.default_rng(3), b, kc, vc)
    if b.num_dec:
        o1 = orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale)
        o2 = orc.decode(b.q_dec, kc2, vc2, t2["tables_dec"], b.lens_dec, b.scale)
        assert np.array_equal(o1, o2), "decode not invariant under relabelling"
    if b.num_pf:
        o1 = orc.prefill(b.q_pf, b.cu_q_lens, kc, vc, b.tables_pf, b.lens_pf, b.scale)
        o2 = orc.prefill(b.q_pf, b.cu_q_lens, kc2, vc2, t2["tables_pf"], b.lens_pf, b.scale)
        assert np.array_equal(o1, o2), "prefill not invariant under relabelling"


def unshare_blocks(b: W.Batch, kc, vc):
    """Gives every sequence private copies of the blocks it shares."""
    tab = b.tables_dec.copy()
    shared = [int(x) for x in b.extra["shared_blocks"]]
    bs = b.spec.block_size
    extra_k, extra_v = [], []
    nxt = kc.shape[0]
    for s in range(b.num_dec):
        for j in range(W.cdiv(int(b.lens_dec[s]), bs)):
            p = int(tab[s, j])
            if p in shared:
                extra_k.append(kc[p])
                extra_v.append(vc[p])
                tab[s, j] = nxt
                nxt += 1
    if extra_k:
        kc = np.concatenate([kc, np.stack(extra_k)])
        vc = np.concatenate([vc, np.stack(extra_v)])
    return kc, vc, tab, len(extra_k)


def pin_sharing_invariance(orc, spec):
    b = W.make_batch(spec)
    kc, vc = appended(orc, b)
    kc2, vc2, tab2, ncopies = unshare_blocks(b, kc, vc)
    assert ncopies > 0
    o1 = orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale)
    o2 = orc.decode(b.q_dec, kc2, vc2, tab2, b.lens_dec, b.scale)
    assert np.array_equal(o1, o2), "decode differs with private copies"


def pin_shared_prefix_diagram(orc):
    g = golden("shared_prefix_diagram.json")
    bs = g["block_size"]
    rng = np.random.default_rng(11)
    Hq, Hkv, D = 4, 2, 16
    NB = 10
    kc = rng.standard_normal((NB, Hkv, bs, D)).astype(np.float16)
    vc = rng.standard_normal((NB, Hkv, bs, D)).astype(np.float16)
    for src, dst in zip(g["shared_blocks"], g["private_copies_of_shared"]):
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    t_shared = np.array([g["tables"]["R1"], g["tables"]["R2"]], np.int32)
    t_priv = t_shared.copy()
    t_priv[1, :3] = g["private_copies_of_shared"]
    lens = np.array([5 * bs - 3, 5 * bs], np.int32)
    q = rng.standard_normal((2, Hq, D)).astype(np.float16)
    o1 = orc.decode(q, kc, vc, t_shared, lens, 0.25)
    o2 = orc.decode(q, kc, vc, t_priv, lens, 0.25)
    assert np.array_equal(o1, o2), "shared-prefix diagram"
    # the shared blocks really are what both requests read first
    for r in range(2):
        L = int(lens[r])
        k = kc[t_shared[r]].transpose(0, 2, 1, 3).reshape(-1, Hkv, D)[:L]
        v = vc[t_shared[r]].transpose(0, 2, 1, 3).reshape(-1, Hkv, D)[:L]
        ref = sdpa(q[r:r + 1], k, v, 0.25)[0]
        assert np.max(np.abs(o1[r] - ref)) < 1e-12, "shared-prefix diagram dense"


def pin_page_table_diagram(orc):
    """For each listed token, only that token's key matches the query, so the
    output is the value stored at the (page, offset) the fixture names."""
    g = golden("page_table_diagram.json")
    bs, NP = g["block_size"], g["num_pages"]
    D = 8
    for req, n, page, off in g["token_locations"]:
        kc = np.zeros((NP, 1, bs, D), np.float16)
        vc = np.zeros((NP, 1, bs, D), np.float16)
        for fp in g["free_pages"]:
            kc[fp] = np.nan
            vc[fp] = np.nan
        kc[page, 0, off] = 4.0
        vc[page, 0, off] = np.arange(1, D + 1)
        pages = g["requests"][req]["pages"]
        table = np.array([pages + [0] * (4 - len(pages))], np.int32)
        q = np.full((1, 1, D), 4.0, np.float16)
        o = orc.decode(q, kc, vc, table, np.array([n], np.int32), 1.0)
        # the marked token's score is 128 above every other token's (0)
        assert np.max(np.abs(o[0, 0] - np.arange(1, D + 1))) < 1e-9, (req, n)
        if n > 1:
            # one token shorter, the marked token is out of reach: all the
            # values seen are zero
            o = orc.decode(q, kc, vc, table, np.array([n - 1], np.int32), 1.0)
            assert np.max(np.abs(o[0, 0])) == 0.0, (req, n, "seen too early")


def pin_append_golden(orc):
    g = golden("kv_append_tiny.json")
    NB, Hkv, bs, D = g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"]
    key = np.array(g["key"], np.float16)
    val = key + np.float16(g["value_offset"])
    kc = np.zeros((NB, Hkv, bs, D), np.float16)
    vc = np.zeros((NB, Hkv, bs, D), np.float16)
    kc2, vc2 = orc.kv_append(key, val, kc, vc, np.array(g["slot_mapping"], np.int32))
    exp = np.zeros(NB * Hkv * bs * D, np.float16)
    for i, x in g["expected_k_nonzero"].items():
        exp[int(i)] = x
    assert np.array_equal(kc2.reshape(-1), exp), "kv_append golden (K)"
    expv = np.where(exp != 0, exp + np.float16(g["value_offset"]), 0).astype(np.float16)
    assert np.array_equal(vc2.reshape(-1), expv), "kv_append golden (V)"


def pin_append_roundtrip(orc, spec):
    """After the append, reading each sequence through its table in logical
    order gives back the generator's logical-order rows, bit for bit, and
    every slot that no new row targets is unchanged."""
    b = W.make_batch(spec, keep_dense=True, pad_rows=3)
    kc, vc = appended(orc, b)
    bs = b.spec.block_size
    seqs = []
    if b.num_dec:
        seqs += [(b.tables_dec[s], int(b.lens_dec[s])) for s in range(b.num_dec)]
    if b.num_pf:
        seqs += [(b.tables_pf[c], int(b.lens_pf[c])) for c in range(b.num_pf)]
    for (row, L), (kd, vd) in zip(seqs, b.dense):
        t = np.arange(L)
        gk = kc[row[t // bs], :, t % bs]
        gv = vc[row[t // bs], :, t % bs]
        assert np.array_equal(gk.view(np.uint16), kd.view(np.uint16)), "K roundtrip"
        assert np.array_equal(gv.view(np.uint16), vd.view(np.uint16)), "V roundtrip"
    touched = np.zeros(kc.shape[0] * bs, bool)
    touched[b.slot_mapping[b.slot_mapping >= 0]] = True
    touched = touched.reshape(kc.shape[0], bs)
    before = b.k_cache.view(np.uint16).transpose(0, 2, 1, 3)[~touched]
    after = kc.view(np.uint16).transpose(0, 2, 1, 3)[~touched]
    assert np.array_equal(before, after), "untouched slots changed"


def pin_swap(orc, spec, seed=5):
    """Swapping ("LLM 推理引擎 …", §4.4: a request's KV goes from its GPU
    blocks to CPU blocks and back) must keep every token's K and V at its
    logical position: after copying each sequence's blocks to shuffled blocks
    of a second pool, decoding through the rewritten tables gives the dense
    attention over the generator's logical-order rows; the second pool's
    other blocks keep their bits; copying the blocks back to fresh positions
    of a third pool gives the same decode, bit for bit."""
    b = W.make_batch(spec, keep_dense=True)
    kc, vc = appended(orc, b)
    NB, Hkv, bs, D = kc.shape
    rng = np.random.default_rng(seed)
    used = [(s, j) for s in range(b.num_dec) for j in range(W.cdiv(int(b.lens_dec[s]), bs))]
    src = np.array(sorted({int(b.tables_dec[s, j]) for s, j in used}), np.int32)
    hNB = len(src) + 5
    dst = rng.permutation(hNB)[:len(src)].astype(np.int32)
    fill = rng.standard_normal((hNB, Hkv, bs, D)).astype(np.float16)
    hk, hv = orc.copy_blocks(kc, vc, fill, fill[::-1].copy(), src, dst)
    where = dict(zip(src.tolist(), dst.tolist()))
    tab = np.zeros_like(b.tables_dec)
    for s, j in used:
        tab[s, j] = where[int(b.tables_dec[s, j])]
    got = orc.decode(b.q_dec, hk, hv, tab, b.lens_dec, b.scale)
    ref = dense_decode_reference(b)
    err = float(np.max(np.abs(got - ref)))
    assert err <= 1e-12, f"{spec.name}: decode after swap-out vs dense {err:.3g}"
    other = np.setdiff1d(np.arange(hNB), dst)
    assert np.array_equal(hk[other].view(np.uint16), fill[other].view(np.uint16)), \
        "blocks outside the copy changed (K)"
    assert np.array_equal(hv[other].view(np.uint16), fill[::-1][other].view(np.uint16)), \
        "blocks outside the copy changed (V)"
    back = rng.permutation(NB)[:len(src)].astype(np.int32)
    zk = np.zeros_like(kc)
    bk, bv = orc.copy_blocks(hk, hv, zk, zk, dst, back)
    where2 = dict(zip(dst.tolist(), back.tolist()))
    tab2 = np.zeros_like(tab)
    for s, j in used:
        tab2[s, j] = where2[int(tab[s, j])]
    got2 = orc.decode(b.q_dec, bk, bv, tab2, b.lens_dec, b.scale)
    assert np.array_equal(got2, got), "swap-in changed the decode"


ALL_PINS = ["half_decoding", "dense_decode", "dense_prefill", "closed_forms",
            "permutation", "sharing", "shared_prefix_diagram",
            "page_table_diagram", "append_golden", "append_roundtrip", "swap"]


def run_pin(orc, name):
    if name == "half_decoding":
        pin_half_decoding(orc)
    elif name == "dense_decode":
        for sp in small_specs():
            pin_dense_decode(orc, sp)
        pin_dense_decode(orc, small_shared_spec())
    elif name == "dense_prefill":
        pin_dense_prefill(orc, small_mixed_spec())
    elif name == "closed_forms":
        pin_closed_forms(orc)
    elif name == "permutation":
        for sp in small_specs()[:3] + [small_mixed_spec()]:
            pin_permutation_invariance(orc, sp)
    elif name == "sharing":
        pin_sharing_invariance(orc, small_shared_spec())
    elif name == "shared_prefix_diagram":
        pin_shared_prefix_diagram(orc)
    elif name == "page_table_diagram":
        pin_page_table_diagram(orc)
    elif name == "append_golden":
        pin_append_golden(orc)
    elif name == "swap":
        for sp in small_specs()[:3]:
            pin_swap(orc, sp)
    elif name == "append_roundtrip":
        for sp in small_specs()[:2] + [small_mixed_spec(), small_shared_spec()]:
            pin_append_roundtrip(orc, sp)
    else:
        raise KeyError(name)
