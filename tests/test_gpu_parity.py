"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: slot writes bit-exact; attention max-abs error <= 2e-3 against the
oracle (fp16 storage, fp32 accumulation).  Tighter diagnostics catch silent
mistakes the bar would hide at long context: decode (fp32 scores, fp32
softmax, fp32 PV) must be within 5e-5; prefill feeds the softmax weights to
the MFMA as fp16 (relative rounding 2^-11 per weight), so its diagnostic is
1e-3.  Invariance under block relabelling and sharing must be bitwise.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_407_amd as pkv
import pins
import workloads as W
from gpu_util import DevBatch, max_abs, say, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 2e-3
TIGHT_DECODE = 5e-5
TIGHT_PREFILL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def gpu_spec(name, Hq, Hkv, D, bs, lens, extra_blocks=9, seed=0):
    nb = sum(W.cdiv(L, bs) for L in lens) + extra_blocks
    return W.Spec(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                  block_size=bs, num_blocks=nb, seed=seed, decode_lens=tuple(lens))


EDGE_LENS = (1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 700)
SMALL_DECODE = [
    gpu_spec("d128_bs16_mha", 4, 4, 128, 16, EDGE_LENS, seed=1),
    gpu_spec("d128_bs32_mha", 2, 2, 128, 32, EDGE_LENS, seed=2),
    gpu_spec("d64_bs16_mha", 4, 4, 64, 16, EDGE_LENS, seed=3),
    gpu_spec("d64_bs32_gqa2", 4, 2, 64, 32, EDGE_LENS, seed=4),
    gpu_spec("d128_bs16_gqa4", 8, 2, 128, 16, EDGE_LENS, seed=5),
    gpu_spec("d128_bs32_gqa8", 16, 2, 128, 32, EDGE_LENS, seed=6),
    # block sizes below one wave-wide load (per-lane block ids) and block
    # size 8, for the decode's block-size sweep
    gpu_spec("d128_bs1_mha", 4, 4, 128, 1, EDGE_LENS, seed=7),
    gpu_spec("d64_bs1_gqa8", 8, 1, 64, 1, EDGE_LENS, seed=8),
    gpu_spec("d128_bs8_gqa2", 4, 2, 128, 8, EDGE_LENS, seed=9),
    gpu_spec("d128_bs8_gqa8", 16, 2, 128, 8, EDGE_LENS, seed=10),
    gpu_spec("d64_bs8_mha", 4, 4, 64, 8, EDGE_LENS, seed=16),
    # 8 query heads per KV head on the matrix cores: both head dims, both
    # block sizes with 16-row tiles
    gpu_spec("d128_bs16_gqa8", 16, 2, 128, 16, EDGE_LENS, seed=18),
    gpu_spec("d64_bs16_gqa8", 8, 1, 64, 16, EDGE_LENS, seed=19),
    gpu_spec("d64_bs32_gqa8", 16, 2, 64, 32, EDGE_LENS, seed=20),
    gpu_spec("d64_bs8_gqa8", 8, 1, 64, 8, EDGE_LENS, seed=22),
    # 16 query heads per KV head: one matrix-core workgroup per KV head
    gpu_spec("d128_bs32_gqa16", 32, 2, 128, 32, EDGE_LENS, seed=23),
    gpu_spec("d64_bs8_gqa16", 16, 1, 64, 8, EDGE_LENS, seed=24),
    # 4 query heads per KV head also run on the matrix cores
    gpu_spec("d64_bs8_gqa4", 8, 2, 64, 8, EDGE_LENS, seed=25),
    # partitions of up to 256 blocks: lengths around 64, 128 and 192 blocks
    # at block size 16 (matrix cores) and up to 256 blocks at block size 8
    # (vector ALUs)
    gpu_spec("d128_bs16_gqa8_long", 16, 2, 128, 16,
             (1, 1023, 1024, 1025, 1040, 2047, 2048, 2049, 3000, 3073, 4096), seed=27),
    gpu_spec("d64_bs8_mha_long", 4, 4, 64, 8, (1, 511, 512, 513, 1024, 1536, 2000, 2048),
             seed=28),
]


def oracle_rows(n_rows, limit, seed=0):
    """All rows (limit None or at least n_rows), or a seeded sample of
    ``limit`` rows (first and last kept)."""
    if limit is None or n_rows <= limit:
        return None
    rng = np.random.default_rng(seed)
    rows = rng.choice(n_rows, size=limit - 2, replace=False)
    return np.unique(np.concatenate([[0, n_rows - 1], rows]))


def check_append(b: W.Batch, dev: DevBatch):
    kc, vc = oracle.kv_append(b.new_k, b.new_v, b.k_cache, b.v_cache, b.slot_mapping)
    gk, gv = to_host(dev.k_cache), to_host(dev.v_cache)
    assert np.array_equal(gk.view(np.uint16), kc.view(np.uint16)), "K pool differs"
    assert np.array_equal(gv.view(np.uint16), vc.view(np.uint16)), "V pool differs"
    return kc, vc


def check_decode(b, kc, vc, got, limit=None, tight=TIGHT_DECODE):
    S, Hq, D = b.q_dec.shape
    rows = oracle_rows(S * Hq, limit)
    ref = oracle.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale, rows=rows)
    g = got.reshape(S * Hq, D)
    r = ref.reshape(S * Hq, D)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert not np.isnan(g).any(), "NaN in decode output"
    err = max_abs(g, r)
    rel = err / float(np.sqrt(np.mean(r ** 2)))
    say(f"decode {b.spec.name}: max-abs {err:.3g} (rel to rms {rel:.3g}) rows "
        f"{'all' if rows is None else len(rows)}")
    assert err <= TOL
    assert err <= tight
    return err


def check_prefill(b, kc, vc, got, limit=None, tight=TIGHT_PREFILL):
    T, Hq, D = b.q_pf.shape
    rows = oracle_rows(T * Hq, limit)
    ref = oracle.prefill(b.q_pf, b.cu_q_lens, kc, vc, b.tables_pf, b.lens_pf, b.scale,
                         rows=rows)
    g = got.reshape(T * Hq, D)
    r = ref.reshape(T * Hq, D)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert not np.isnan(g).any(), "NaN in prefill output"
    err = max_abs(g, r)
    rel = err / float(np.sqrt(np.mean(r ** 2)))
    say(f"prefill {b.spec.name}: max-abs {err:.3g} (rel to rms {rel:.3g}) rows "
        f"{'all' if rows is None else len(rows)}")
    assert err <= TOL
    assert err <= tight
    return err


# ------------------------------------------------------------------ kv append
@pytest.mark.parametrize("name", ["tiny", "llama_decode", "mixed", "gqa_shared"])
def test_append_bit_exact(name):
    say("append", name)
    b = W.make_batch(name, pad_rows=5)
    dev = DevBatch(b)
    dev.append()
    torch.cuda.synchronize()
    check_append(b, dev)


def test_append_skips_out_of_pool_slot():
    b = W.make_batch("tiny")
    dev = DevBatch(b)
    slots = b.slot_mapping.copy()
    slots[0] = b.spec.num_blocks * b.spec.block_size + 3  # beyond the pool
    dev.slots = to_dev(slots)
    dev.append()
    keep = slots.copy()
    keep[0] = -1
    kc, vc = oracle.kv_append(b.new_k, b.new_v, b.k_cache, b.v_cache, keep)
    assert np.array_equal(to_host(dev.k_cache).view(np.uint16), kc.view(np.uint16))


def test_append_zero_tokens():
    b = W.make_batch("tiny")
    dev = DevBatch(b)
    import paged_kv_cache_407_amd as pkv
    e = torch.empty((0,) + tuple(dev.new_k.shape[1:]), dtype=torch.float16, device="cuda")
    pkv.kv_append(e, e, dev.k_cache, dev.v_cache, torch.empty(0, dtype=torch.int32, device="cuda"))
    assert np.array_equal(to_host(dev.k_cache).view(np.uint16), b.k_cache.view(np.uint16))


# --------------------------------------------------------------------- decode
@pytest.mark.parametrize("name", ["tiny", "llama_decode", "gqa_shared", "gqa4", "gqa16"])
def test_decode_config(name):
    # every output element of the batch against the oracle
    say("decode", name)
    b = W.make_batch(name)
    dev = DevBatch(b)
    dev.append()
    out = to_host(dev.decode())
    kc, vc = check_append(b, dev)
    check_decode(b, kc, vc, out)


def max_partition(spec):
    """Largest partition the decode takes: 256 blocks (four block ids per
    lane), 64 at block size 1."""
    return (256 if spec.block_size >= 8 else 64) * spec.block_size


@pytest.mark.parametrize("spec", SMALL_DECODE, ids=lambda s: s.name)
@pytest.mark.parametrize("part", [0, None, 64, "max"])
def test_decode_edge_lengths(spec, part):
    # part None = one partition per block (the smallest split); "max" = the
    # largest partition (block ids past the first 64 of a partition)
    part = spec.block_size if part is None else max_partition(spec) if part == "max" else part
    say("decode edges", spec.name, "partition", part)
    b = W.make_batch(spec, pad_rows=2)
    dev = DevBatch(b)
    dev.append()
    out = to_host(dev.decode(partition_size=part))
    kc, vc = check_append(b, dev)
    check_decode(b, kc, vc, out)


def _random_decode_cases(n=16, seed=777):
    """Seeded random shapes over the decode's routing: head dim 64 or 128,
    block size 1, 8, 16 or 32, 1 to 16 query heads per KV head (vector-ALU
    and matrix-core kernels, 4, 8 and 16 heads per workgroup), 3 to 40
    sequences with log-uniform lengths that include 1 and block boundaries,
    and a partition size of the library's choice, one block, or a random
    multiple of the block size up to the largest; every other case is
    dispatched in a random order."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        bs = int(rng.choice([1, 8, 16, 32]))
        hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        n_seqs = int(rng.integers(3, 41))
        hi = 4096 if bs >= 8 else 1024
        lens = np.exp(rng.uniform(0.0, np.log(hi), n_seqs)).astype(int).clip(1, hi)
        lens[0] = 1
        lens[1] = bs * int(rng.integers(1, 9))  # a full last block
        spec = gpu_spec(f"dec_rand{i}_d{D}_bs{bs}_{hkv * G}x{hkv}_s{n_seqs}", hkv * G, hkv, D,
                        bs, tuple(int(L) for L in lens), seed=6000 + i)
        top = max_partition(spec) // bs
        part = [0, bs, bs * int(rng.integers(1, top + 1))][i % 3]
        order = rng.permutation(n_seqs).astype(np.int32) if i % 2 else None
        cases.append((spec, part, order))
    return cases


@pytest.mark.parametrize("spec,part,order", _random_decode_cases(),
                         ids=lambda c: c.name if isinstance(c, W.Spec) else None)
def test_decode_random_shapes(spec, part, order):
    say("decode random", spec.name, "partition", part,
        "order", "given" if order is not None else "none")
    b = W.make_batch(spec, pad_rows=2)
    dev = DevBatch(b)
    dev.append()
    out = to_host(dev.decode(partition_size=part, seq_order=order))
    kc, vc = check_append(b, dev)
    check_decode(b, kc, vc, out)


def test_decode_long_context():
    # both 4 GiB pools bitwise after the append, every output row
    say("decode long (8 x 32768)")
    b = W.make_batch("long")
    dev = DevBatch(b)
    dev.append()
    out = to_host(dev.decode())
    kc, vc = check_append(b, dev)
    check_decode(b, kc, vc, out)


def test_decode_split_matches_unsplit():
    say("decode split vs unsplit")
    b = W.make_batch("llama_decode")
    dev = DevBatch(b)
    dev.append()
    one = to_host(dev.decode(partition_size=1024))   # a single partition
    for part in (16, 64, 256, 512):
        split = to_host(dev.decode(partition_size=part))
        err = max_abs(split, one)
        say(f"partition {part}: {err:.3g}")
        assert err <= 1e-6


@pytest.mark.parametrize("name", ["llama_decode", "gqa_shared", "tiny"])
def test_decode_dispatch_order_is_bitwise_neutral(name):
    # the dispatch order only changes when a sequence runs, never its result
    say("decode dispatch order", name)
    b = W.make_batch(name)
    dev = DevBatch(b)
    dev.append()
    base = to_host(dev.decode())
    orders = [pkv.longest_first(b.lens_dec),
              np.random.default_rng(3).permutation(b.num_dec).astype(np.int32)]
    for order in orders:
        got = to_host(dev.decode(seq_order=order))
        assert np.array_equal(got.view(np.uint32), base.view(np.uint32))
    kc, vc = check_append(b, dev)
    check_decode(b, kc, vc, to_host(dev.decode(seq_order=orders[0])))


# 8 query heads per KV head at block size 32 with a shared prefix: the
# matrix-core decode, small enough to relabel on the host
GQA_PERM = W.Spec(name="gqa_perm", num_q_heads=16, num_kv_heads=2, head_dim=128,
                  block_size=32, num_blocks=640, seed=21, decode_count=24,
                  decode_dist="uniform", decode_lo=20, decode_hi=700, shared_prefix=64)


@pytest.mark.parametrize("spec,part", [("llama_decode", 0), (GQA_PERM, 0), (GQA_PERM, 64)],
                         ids=["llama_decode", "gqa8_bs32", "gqa8_bs32_split"])
def test_decode_permutation_invariance_bitwise(spec, part):
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    o1 = to_host(dev.decode(partition_size=part))
    kc, vc = to_host(dev.k_cache), to_host(dev.v_cache)
    kc2, vc2, t2 = pins.relabel_blocks(np.random.default_rng(5), b, kc, vc)
    o2 = to_host(dev.decode(partition_size=part, tables=to_dev(t2["tables_dec"]),
                            k_cache=to_dev(kc2), v_cache=to_dev(vc2)))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    if spec is GQA_PERM:
        check_decode(b, kc, vc, o1)


def test_decode_sharing_invariance_bitwise():
    # the shared-prefix structure at a supported shape (D=64, bs=16)
    spec = W.Spec(name="shared_gpu", num_q_heads=16, num_kv_heads=2, head_dim=64,
                  block_size=16, num_blocks=512, seed=8, decode_count=12,
                  decode_dist="uniform", decode_lo=20, decode_hi=300, shared_prefix=64)
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    o1 = to_host(dev.decode(partition_size=64))
    kc, vc = to_host(dev.k_cache), to_host(dev.v_cache)
    kc2, vc2, tab2, n = pins.unshare_blocks(b, kc, vc)
    assert n > 0
    o2 = to_host(dev.decode(partition_size=64, tables=to_dev(tab2), k_cache=to_dev(kc2),
                            v_cache=to_dev(vc2)))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


GQA16_BS8 = gpu_spec("d128_bs8_gqa16", 32, 2, 128, 8, (1, 17, 200, 700, 33, 64, 300, 129),
                     seed=26)


MHA_BS8_LONG = gpu_spec("mha_bs8_long", 4, 4, 64, 8, (1, 600, 1000, 1700, 2000, 2048), seed=29)


@pytest.mark.parametrize("spec,parts", [("llama_decode", (0, 1024)), (GQA_PERM, (0, 64)),
                                        (GQA16_BS8, (0, 64, 1024)),
                                        (MHA_BS8_LONG, (0, 2048))],
                         ids=["llama_decode", "gqa8_bs32", "gqa16_bs8", "mha_bs8_long"])
def test_decode_bad_rows_are_nan_and_others_unaffected(spec, parts):
    # an out-of-pool block id, an empty sequence and a length beyond the
    # host bound poison their own rows only; on the vector-ALU kernel (MHA)
    # and the matrix-core kernel (8 and 16 query heads per KV head; at block
    # size 8 with 1024-token partitions, also a bad id among a partition's
    # blocks 64..127)
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    bs = b.spec.block_size
    long_seqs = [s for s in range(b.num_dec) if b.lens_dec[s] > bs]
    s_blk = long_seqs[0]
    tab = b.tables_dec.copy()
    tab[s_blk, 1] = b.spec.num_blocks + 7   # out-of-range block id
    bad = [s_blk]
    # out-of-range ids past the first 64 and past the first 192 of a
    # partition (second and fourth id register), in other sequences
    for j in (70, 200):
        cand = [s for s in range(b.num_dec) if b.lens_dec[s] > (j + 1) * bs and s not in bad]
        if cand:
            tab[cand[0], j] = -3
            bad.append(cand[0])
    s_zero, s_big = [s for s in range(b.num_dec) if s not in bad][:2]
    lens = b.lens_dec.copy()
    lens[s_zero] = 0                        # empty sequence
    lens[s_big] = dev.max_len_dec + 1       # beyond the host bound
    bad = tuple(bad) + (s_zero, s_big)
    others = [s for s in range(b.num_dec) if s not in bad]
    for part in parts:
        good = to_host(dev.decode(partition_size=part))
        out = to_host(dev.decode(partition_size=part, tables=to_dev(tab), lens=to_dev(lens)))
        for s in bad:
            assert np.isnan(out[s]).all(), (part, s)
        assert np.array_equal(out[others].view(np.uint32), good[others].view(np.uint32))


def test_decode_empty_batch():
    import paged_kv_cache_407_amd as pkv
    kc = torch.zeros((4, 2, 16, 64), dtype=torch.float16, device="cuda")
    q = torch.zeros((0, 2, 64), dtype=torch.float16, device="cuda")
    t = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    lens = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out = pkv.paged_attention_decode(q, kc, kc, t, lens, max_seq_len=64)
    assert out.shape == (0, 2, 64)


# -------------------------------------------------------------------- prefill
def pf_spec(name, Hq, Hkv, D, bs, chunk, prefix_hi, n_chunks=3, seed=0):
    mb = max(40, W.cdiv(600, bs), W.cdiv(chunk + prefix_hi, bs))
    return W.Spec(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                  num_blocks=n_chunks * W.cdiv(chunk + prefix_hi, bs) + 4 * mb + 9,
                  seed=seed, decode_count=4, decode_dist="uniform", decode_lo=1,
                  decode_hi=600, prefill_chunks=n_chunks, prefill_chunk_len=chunk,
                  prefill_prefix_lo=0, prefill_prefix_hi=prefix_hi, max_blocks_per_seq=mb)


SMALL_PREFILL = [
    pf_spec("pf_d128_bs16", 4, 4, 128, 16, 100, 200, seed=11),
    pf_spec("pf_d128_bs32_gqa", 8, 2, 128, 32, 64, 130, seed=12),
    pf_spec("pf_d64_bs16", 4, 4, 64, 16, 1, 300, seed=13),
    pf_spec("pf_d64_bs32", 4, 1, 64, 32, 129, 0, seed=14),
    pf_spec("pf_d128_bs16_long", 2, 2, 128, 16, 300, 300, seed=15),
    pf_spec("pf_d128_bs8_gqa", 4, 2, 128, 8, 100, 200, seed=17),
    pf_spec("pf_d64_bs8", 4, 4, 64, 8, 130, 70, seed=18),
    # 8 and 16 query heads per KV head
    pf_spec("pf_d128_bs16_gqa8", 16, 2, 128, 16, 90, 250, seed=19),
    pf_spec("pf_d64_bs32_gqa16", 16, 1, 64, 32, 140, 100, seed=20),
]


@pytest.mark.parametrize("spec", SMALL_PREFILL, ids=lambda s: s.name)
def test_prefill_small(spec):
    say("prefill", spec.name)
    b = W.make_batch(spec, pad_rows=3)
    dev = DevBatch(b)
    dev.append()
    out = to_host(dev.prefill())
    kc, vc = check_append(b, dev)
    check_prefill(b, kc, vc, out)
    dec = to_host(dev.decode())
    check_decode(b, kc, vc, dec)


def _random_prefill_specs(n=12, seed=4242):
    """Seeded random shapes over every compiled prefill instance: head dim
    64 or 128, block size 8, 16 or 32, 1 to 4 query heads per KV head, 1 to
    4 chunks whose lengths and prefixes fall anywhere relative to the 128-row
    query tiles and 64-key tiles; every third case has prefixes long enough
    for the key range to be split across workgroups."""
    rng = np.random.default_rng(seed)
    specs = []
    for i in range(n):
        D = int(rng.choice([64, 128]))
        bs = int(rng.choice([8, 16, 32]))
        hkv = int(rng.choice([1, 2, 4]))
        hq = hkv * int(rng.choice([1, 2, 4]))
        chunk = int(rng.integers(1, 300))
        prefix = int(rng.integers(1100, 2600)) if i % 3 == 2 else int(rng.integers(0, 400))
        n_chunks = int(rng.integers(1, 5))
        specs.append(pf_spec(f"pf_rand{i}_d{D}_bs{bs}_{hq}x{hkv}_c{chunk}_p{prefix}_n{n_chunks}",
                             hq, hkv, D, bs, chunk, prefix, n_chunks=n_chunks, seed=5000 + i))
    return specs


@pytest.mark.parametrize("spec", _random_prefill_specs(), ids=lambda s: s.name)
def test_prefill_random_shapes(spec):
    say("prefill random", spec.name)
    b = W.make_batch(spec, pad_rows=2)
    dev = DevBatch(b)
    dev.append()
    out = to_host(dev.prefill())
    kc, vc = check_append(b, dev)
    check_prefill(b, kc, vc, out)


def test_prefill_ragged_chunks():
    say("prefill ragged")
    spec = pf_spec("pf_ragged", 4, 2, 128, 16, 64, 100, n_chunks=4, seed=21)
    b = W.make_batch(spec)
    # cut the 4 equal chunks into lengths 1, 63, 65, 127 by moving rows around:
    # rebuild q / cu / lens for chunks whose new tokens are a prefix of the
    # generated ones, so every row keeps its generated key.
    lens_c = np.array([1, 63, 64, 17], np.int64)
    keep_rows, cu = [], [0]
    new_lens = []
    for c in range(4):
        lo = int(b.cu_q_lens[c])
        keep_rows.extend(range(lo, lo + int(lens_c[c])))
        cu.append(cu[-1] + int(lens_c[c]))
        prefix = int(b.lens_pf[c]) - 64
        new_lens.append(prefix + int(lens_c[c]))
    b.q_pf = b.q_pf[keep_rows]
    b.cu_q_lens = np.array(cu, np.int32)
    b.lens_pf = np.array(new_lens, np.int32)
    dev = DevBatch(b)
    dev.append()   # appends all 64 rows per chunk; the extra rows are unseen
    out = to_host(dev.prefill())
    kc, vc = oracle.kv_append(b.new_k, b.new_v, b.k_cache, b.v_cache, b.slot_mapping)
    check_prefill(b, kc, vc, out)


def test_prefill_mixed_config():
    say("mixed step")
    b = W.make_batch("mixed")
    dev = DevBatch(b)
    dev.append()
    pf = to_host(dev.prefill())
    dec = to_host(dev.decode())
    kc, vc = check_append(b, dev)
    # every prefill and decode output element against the oracle
    check_prefill(b, kc, vc, pf)
    check_decode(b, kc, vc, dec)


def test_prefill_last_row_matches_decode():
    spec = pf_spec("pf_vs_dec", 4, 4, 128, 16, 80, 150, seed=31)
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    pf = to_host(dev.prefill())
    # decode the chunks' sequences with the chunk's last query row
    import paged_kv_cache_407_amd as pkv
    last = b.cu_q_lens[1:] - 1
    out = pkv.paged_attention_decode(
        to_dev(b.q_pf[last]), dev.k_cache, dev.v_cache, dev.tables_pf, dev.lens_pf,
        max_seq_len=int(b.lens_pf.max()), scale=b.scale)
    err = max_abs(to_host(out), pf[last])
    say(f"last prefill row vs decode: {err:.3g}")
    assert err <= TOL


def test_prefill_permutation_invariance_bitwise():
    spec = pf_spec("pf_perm", 4, 4, 128, 16, 100, 200, seed=41)
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    o1 = to_host(dev.prefill())
    kc, vc = to_host(dev.k_cache), to_host(dev.v_cache)
    kc2, vc2, t2 = pins.relabel_blocks(np.random.default_rng(6), b, kc, vc)
    o2 = to_host(dev.prefill(tables=to_dev(t2["tables_pf"]), k_cache=to_dev(kc2),
                             v_cache=to_dev(vc2)))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_prefill_bad_chunk_is_nan():
    spec = pf_spec("pf_bad", 4, 4, 128, 16, 70, 100, seed=51)
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    good = to_host(dev.prefill())
    tab = b.tables_pf.copy()
    tab[1, 0] = -5
    out = to_host(dev.prefill(tables=to_dev(tab)))
    lo, hi = int(b.cu_q_lens[1]), int(b.cu_q_lens[2])
    assert np.isnan(out[lo:hi]).all()
    rest = np.r_[0:lo, hi:out.shape[0]]
    assert np.array_equal(out[rest].view(np.uint32), good[rest].view(np.uint32))


# ------------------------------------------------- split key ranges (prefill)
# Few query tiles on long prefixes: the library cuts each query tile's key
# range into parts run by different workgroups and merges them.  The chunk on
# an empty prefix has too few key tiles to split and is written directly in
# the same launch.
SPLIT_PREFIXES = [2000, 0, 900, 1500]
SPLIT_CHUNK = 70


def split_spec(D, bs, Hq, Hkv, seed):
    L = [p + SPLIT_CHUNK for p in SPLIT_PREFIXES]
    return W.Spec(name=f"split_d{D}_bs{bs}_{Hq}_{Hkv}", num_q_heads=Hq, num_kv_heads=Hkv,
                  head_dim=D, block_size=bs,
                  num_blocks=sum(W.cdiv(x, bs) for x in L) + 2 * W.cdiv(100, bs) + 16,
                  seed=seed, decode_count=2, decode_dist="uniform", decode_lo=1, decode_hi=100,
                  prefill_chunks=len(L), prefill_chunk_len=SPLIT_CHUNK,
                  max_blocks_per_seq=W.cdiv(max(L), bs))


def split_call(b, dev, max_seq_len, tables=None, workspace=None):
    return to_host(pkv.paged_attention_prefill(
        dev.q_pf, dev.cu, dev.k_cache, dev.v_cache,
        dev.tables_pf if tables is None else tables, dev.lens_pf, max_q_len=SPLIT_CHUNK,
        max_seq_len=max_seq_len, scale=b.scale, workspace=workspace))


@pytest.mark.parametrize("D,bs,Hq,Hkv", [(128, 16, 2, 1), (64, 8, 4, 4), (128, 32, 4, 2),
                                         (128, 8, 2, 2), (64, 16, 2, 1)],
                         ids=lambda x: str(x))
def test_prefill_split_key_ranges(D, bs, Hq, Hkv):
    spec = split_spec(D, bs, Hq, Hkv, seed=D + bs + Hq)
    say("prefill split", spec.name)
    b = W.make_batch(spec, lens_override={"prefix": SPLIT_PREFIXES})
    T = b.q_pf.shape[0]
    maxl = int(b.lens_pf.max())
    need = pkv.prefill_workspace_size(len(SPLIT_PREFIXES), T, SPLIT_CHUNK, Hq, D, maxl)
    assert need > 0                      # the call takes the split path
    dev = DevBatch(b)
    dev.append()
    kc, vc = check_append(b, dev)
    # a workspace holding NaN bit patterns: its contents on entry do not matter
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = split_call(b, dev, maxl, workspace=ws)
    check_prefill(b, kc, vc, out)
    # a looser bound on the lengths cuts the key ranges differently
    out2 = split_call(b, dev, spec.max_blocks_per_seq * bs)
    check_prefill(b, kc, vc, out2)
    # the same call again on the same workspace is bitwise repeatable
    assert np.array_equal(split_call(b, dev, maxl, workspace=ws).view(np.uint32),
                          out.view(np.uint32))


def test_prefill_split_bad_block_and_short_bound():
    spec = split_spec(128, 16, 2, 1, seed=77)
    b = W.make_batch(spec, lens_override={"prefix": SPLIT_PREFIXES})
    dev = DevBatch(b)
    dev.append()
    maxl = int(b.lens_pf.max())
    good = split_call(b, dev, maxl)
    cu = b.cu_q_lens
    rows = lambda c: np.r_[int(cu[c]):int(cu[c + 1])]
    # an out-of-range block id in the middle of chunk 0's prefix (one part of
    # its split key range) turns the chunk's rows to NaN, nothing else
    tab = b.tables_pf.copy()
    tab[0, 60] = spec.num_blocks + 5
    bad = split_call(b, dev, maxl, tables=to_dev(tab))
    assert np.isnan(bad[rows(0)]).all()
    rest = np.r_[int(cu[1]):bad.shape[0]]
    assert np.array_equal(bad[rest].view(np.uint32), good[rest].view(np.uint32))
    # chunks longer than max_seq_len get NaN rows; the others stay exact
    short = split_call(b, dev, 1000)
    kc, vc = to_host(dev.k_cache), to_host(dev.v_cache)
    for c, L in enumerate(b.lens_pf):
        if L > 1000:
            assert np.isnan(short[rows(c)]).all()
        else:
            assert not np.isnan(short[rows(c)]).any()
    keep = [c for c, L in enumerate(b.lens_pf) if L <= 1000]
    ref = oracle.prefill(b.q_pf, b.cu_q_lens, kc, vc, b.tables_pf, b.lens_pf, b.scale)
    for c in keep:
        assert max_abs(short[rows(c)], ref[rows(c)]) <= TOL
    # a workspace below the size the call needs is refused
    need = pkv.prefill_workspace_size(4, b.q_pf.shape[0], SPLIT_CHUNK, 2, 128, maxl)
    with pytest.raises(pkv.PkvError):
        split_call(b, dev, maxl, workspace=torch.empty(need - 256, dtype=torch.uint8,
                                                      device="cuda"))


# --------------------------------------------- grouped heads, workspace reuse
@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (12, 2), (12, 1), (16, 1), (6, 6)],
                         ids=lambda x: str(x))
def test_decode_head_groups(Hq, Hkv):
    # group sizes 3, 6, 12, 16, 1: one query head per workgroup (vector ALUs)
    # for 3 and 1, two for 6, four for 12 and sixteen for 16 (matrix cores)
    spec = gpu_spec(f"groups_{Hq}_{Hkv}", Hq, Hkv, 128, 16, (1, 17, 200, 700), seed=Hq * 7 + Hkv)
    say("decode head groups", spec.name)
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    kc, vc = check_append(b, dev)
    for part in (0, 64):
        check_decode(b, kc, vc, to_host(dev.decode(partition_size=part)))


def test_decode_workspace_reuse_across_shapes():
    # one workspace serves calls with different splits; stale partials of an
    # earlier layout never leak into a later call
    import paged_kv_cache_407_amd as pkv
    say("decode workspace reuse")
    b = W.make_batch("llama_decode")
    dev = DevBatch(b)
    dev.append()
    kc, vc = check_append(b, dev)
    spec = b.spec
    need = max(pkv.decode_workspace_size(b.num_dec, spec.num_q_heads, spec.num_kv_heads,
                                         spec.head_dim, spec.block_size, dev.max_len_dec, part)
               for part in (0, 64, 128))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    first = None
    for part in (0, 64, 128, 0):
        out = torch.full((b.num_dec, spec.num_q_heads, spec.head_dim), float("nan"),
                         dtype=torch.float32, device="cuda")
        pkv.paged_attention_decode(dev.q_dec, dev.k_cache, dev.v_cache, dev.tables_dec,
                                   dev.lens_dec, max_seq_len=dev.max_len_dec, scale=b.scale,
                                   out=out, workspace=ws, partition_size=part)
        o = to_host(out)
        check_decode(b, kc, vc, o)
        if part == 0:
            if first is None:
                first = o
            assert np.array_equal(o.view(np.uint32), first.view(np.uint32))


@pytest.mark.parametrize("name", ["llama_decode", "gqa_shared"])
def test_decode_graph_replays_match_eager(name):
    say("decode graph replays")
    b = W.make_batch(name)
    dev = DevBatch(b)
    dev.append()
    import paged_kv_cache_407_amd as pkv
    spec = b.spec
    need = pkv.decode_workspace_size(b.num_dec, spec.num_q_heads, spec.num_kv_heads,
                                     spec.head_dim, spec.block_size, dev.max_len_dec)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out = torch.empty((b.num_dec, spec.num_q_heads, spec.head_dim), dtype=torch.float32,
                      device="cuda")

    def run():
        pkv.paged_attention_decode(dev.q_dec, dev.k_cache, dev.v_cache, dev.tables_dec,
                                   dev.lens_dec, max_seq_len=dev.max_len_dec, scale=b.scale,
                                   out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    eager = to_host(out).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host(out)
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), i


def test_prefill_split_graph_replays_match_eager():
    # the split prefill (parts into the workspace, then the merge kernel)
    # captured in a HIP graph: every replay, with other prefill work on the
    # same workspace in between, matches the eager call bit for bit
    spec = split_spec(128, 16, 2, 1, seed=91)
    b = W.make_batch(spec, lens_override={"prefix": SPLIT_PREFIXES})
    dev = DevBatch(b)
    dev.append()
    T, Hq, D = b.q_pf.shape
    maxl = int(b.lens_pf.max())
    need = pkv.prefill_workspace_size(len(SPLIT_PREFIXES), T, SPLIT_CHUNK, Hq, D, maxl)
    loose = spec.max_blocks_per_seq * 16     # a looser bound splits differently
    need2 = pkv.prefill_workspace_size(len(SPLIT_PREFIXES), T, SPLIT_CHUNK, Hq, D, loose)
    assert need > 0 and need2 > 0
    ws = torch.zeros(max(need, need2), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, Hq, D), dtype=torch.float32, device="cuda")

    def run():
        pkv.paged_attention_prefill(dev.q_pf, dev.cu, dev.k_cache, dev.v_cache, dev.tables_pf,
                                    dev.lens_pf, max_q_len=SPLIT_CHUNK, max_seq_len=maxl,
                                    scale=b.scale, out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    eager = to_host(out).copy()
    kc, vc = check_append(b, dev)
    check_prefill(b, kc, vc, eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(4):
        out.fill_(float("nan"))
        split_call(b, dev, loose, workspace=ws)   # another split on the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out).view(np.uint32), eager.view(np.uint32)), i


# ------------------------------------------------------- host block manager
def test_block_manager_drives_append_and_decode():
    """Block tables and slot mappings from the host block manager drive the
    kernels: prompts are written through their slots, one decode step appends
    a token per sequence (some crossing a block boundary), and the decode
    reads the new tokens back through the manager's tables."""
    rng = np.random.default_rng(99)
    Hq, Hkv, D, bs, NB = 8, 2, 128, 16, 256
    lens = [1, 15, 16, 17, 100, 257, 33]
    bm = pkv.BlockManager(NB - 1, bs)      # block NB-1 stays free: the pad canary
    kc = np.full((NB, Hkv, bs, D), np.nan, np.float16)
    vc = np.full((NB, Hkv, bs, D), np.nan, np.float16)
    ids = list(range(len(lens)))
    pk, pv, ps = [], [], []
    for r, L in zip(ids, lens):
        bm.allocate(r, L - 1)
        pk.append(rng.standard_normal((L - 1, Hkv, D)).astype(np.float16))
        pv.append(rng.standard_normal((L - 1, Hkv, D)).astype(np.float16))
        ps.append(bm.slots(r, 0, L - 1))
    pk, pv, ps = np.concatenate(pk), np.concatenate(pv), np.concatenate(ps).astype(np.int32)
    nk = rng.standard_normal((len(ids), Hkv, D)).astype(np.float16)
    nv = rng.standard_normal((len(ids), Hkv, D)).astype(np.float16)
    ns = bm.append_tokens(ids)
    MB = 20
    tables, seq_lens = bm.build_tables(ids, MB, pad_block=NB - 1)
    assert list(seq_lens) == lens
    q = rng.standard_normal((len(ids), Hq, D)).astype(np.float16)
    scale = float(np.float32(1 / np.sqrt(D)))

    dk, dv = to_dev(kc), to_dev(vc)
    pkv.kv_append(to_dev(pk), to_dev(pv), dk, dv, to_dev(ps))
    pkv.kv_append(to_dev(nk), to_dev(nv), dk, dv, to_dev(ns))
    out = to_host(pkv.paged_attention_decode(to_dev(q), dk, dv, to_dev(tables),
                                             to_dev(seq_lens), max_seq_len=max(lens),
                                             scale=scale, partition_size=64))
    okc, ovc = oracle.kv_append(pk, pv, kc, vc, ps)
    okc, ovc = oracle.kv_append(nk, nv, okc, ovc, ns)
    assert np.array_equal(to_host(dk).view(np.uint16), okc.view(np.uint16))
    ref = oracle.decode(q, okc, ovc, tables, seq_lens, scale)
    err = max_abs(out, ref)
    say(f"block manager end to end: max-abs {err:.3g}")
    assert err <= TIGHT_DECODE


# -------------------------------------------------- block copies (swapping)
def _pinned_pool(shape, fill):
    t = torch.empty(shape, dtype=torch.float16, pin_memory=True)
    t.copy_(torch.from_numpy(np.ascontiguousarray(fill).view(np.int16)).view(torch.float16))
    return t


def _pinned_ids(a):
    t = torch.empty(len(a), dtype=torch.int32, pin_memory=True)
    t.copy_(torch.from_numpy(np.asarray(a, np.int32)))
    return t


@pytest.mark.parametrize("ids_on", ["device", "pinned"])
def test_copy_blocks_out_and_back_bit_exact(ids_on):
    """Device pool -> pinned host pool -> fresh device pool, against the
    oracle's block copy; the request's decode survives the round trip bit
    for bit (the same kernel on the same bytes at other block ids)."""
    spec = gpu_spec("swap_d128_bs16", 8, 2, 128, 16, (1, 16, 17, 200, 333), seed=31)
    b = W.make_batch(spec)
    dev = DevBatch(b)
    dev.append()
    before = to_host(dev.decode())
    kc, vc = check_append(b, dev)
    NB, Hkv, bs, D = kc.shape
    rng = np.random.default_rng(7)
    used = [(s, j) for s in range(b.num_dec) for j in range(W.cdiv(int(b.lens_dec[s]), bs))]
    src = np.array([int(b.tables_dec[s, j]) for s, j in used], np.int32)
    hNB = len(src) + 6
    dst = rng.permutation(hNB)[:len(src)].astype(np.int32)
    fill = rng.standard_normal((hNB, Hkv, bs, D)).astype(np.float16)
    hk, hv = _pinned_pool(fill.shape, fill), _pinned_pool(fill.shape, fill[::-1])
    mk = to_dev if ids_on == "device" else _pinned_ids
    say("copy blocks out", len(src), "blocks, ids on", ids_on)
    pkv.copy_blocks(dev.k_cache, dev.v_cache, hk, hv, mk(src), mk(dst))
    torch.cuda.synchronize()
    ok, ov = oracle.copy_blocks(kc, vc, fill, fill[::-1], src, dst)
    assert np.array_equal(hk.numpy().view(np.uint16), ok.view(np.uint16))
    assert np.array_equal(hv.numpy().view(np.uint16), ov.view(np.uint16))
    back = rng.permutation(NB)[:len(src)].astype(np.int32)
    nk = torch.zeros_like(dev.k_cache)
    nv = torch.zeros_like(dev.v_cache)
    say("copy blocks back")
    pkv.copy_blocks(hk, hv, nk, nv, mk(dst), mk(back))
    torch.cuda.synchronize()
    bk, bv = oracle.copy_blocks(ok, ov, np.zeros_like(kc), np.zeros_like(vc), dst, back)
    assert np.array_equal(to_host(nk).view(np.uint16), bk.view(np.uint16))
    assert np.array_equal(to_host(nv).view(np.uint16), bv.view(np.uint16))
    tab = b.tables_dec.copy()
    for (s, j), p in zip(used, back):
        tab[s, j] = p
    after = to_host(dev.decode(tables=to_dev(tab), k_cache=nk, v_cache=nv))
    assert np.array_equal(after.view(np.uint32), before.view(np.uint32))


def test_copy_blocks_dma_matches_kernel():
    """The DMA path (host id lists, one copy per run of consecutive blocks)
    writes the same bytes as the kernel path, device -> device and device
    -> pinned host."""
    rng = np.random.default_rng(8)
    NB, Hkv, bs, D = 64, 4, 16, 64
    pool = rng.standard_normal((2, NB, Hkv, bs, D)).astype(np.float16)
    sk, sv = to_dev(pool[0]), to_dev(pool[1])
    src = np.array([3, 4, 5, 9, 10, 40, 41, 42, 43, 7], np.int32)   # runs of 3, 2, 4, 1
    dst = np.array([20, 21, 22, 0, 1, 50, 51, 52, 53, 63], np.int32)
    for kind in ("device", "pinned"):
        if kind == "device":
            a = [torch.zeros_like(sk) for _ in range(4)]
        else:
            a = [_pinned_pool(pool[0].shape, np.zeros_like(pool[0])) for _ in range(4)]
        say("copy blocks dma vs kernel,", kind, "destination")
        pkv.copy_blocks(sk, sv, a[0], a[1], to_dev(src), to_dev(dst))
        pkv.copy_blocks_dma(sk, sv, a[2], a[3], src, dst)
        torch.cuda.synchronize()
        ref_k, ref_v = oracle.copy_blocks(pool[0], pool[1], np.zeros_like(pool[0]),
                                          np.zeros_like(pool[1]), src, dst)
        for t, r in ((a[0], ref_k), (a[1], ref_v), (a[2], ref_k), (a[3], ref_v)):
            got = to_host(t) if kind == "device" else t.numpy()
            assert np.array_equal(got.view(np.uint16), r.view(np.uint16))


def test_copy_blocks_skips_ids_outside_pools():
    rng = np.random.default_rng(9)
    NB, Hkv, bs, D = 16, 2, 16, 128
    pool = rng.standard_normal((2, NB, Hkv, bs, D)).astype(np.float16)
    sk, sv = to_dev(pool[0]), to_dev(pool[1])
    dk, dv = torch.zeros_like(sk), torch.zeros_like(sv)
    src = np.array([1, -1, 2, 99, 3], np.int32)
    dst = np.array([4, 5, 16, 6, 7], np.int32)
    say("copy blocks with ids outside the pools")
    pkv.copy_blocks(sk, sv, dk, dv, to_dev(src), to_dev(dst))
    torch.cuda.synchronize()
    ok = (src >= 0) & (src < NB) & (dst >= 0) & (dst < NB)
    rk, rv = oracle.copy_blocks(pool[0], pool[1], np.zeros_like(pool[0]), np.zeros_like(pool[1]),
                                src[ok], dst[ok])
    assert np.array_equal(to_host(dk).view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(to_host(dv).view(np.uint16), rv.view(np.uint16))
    with pytest.raises(pkv.PkvError):
        pkv.copy_blocks_dma(sk, sv, dk, dv, src, dst)   # host-checked: rejected


def test_swap_preempted_request_and_resume():
    """The pages' swap flow end to end: a request is swapped out to a pinned
    host pool (block pairs from the block managers), its GPU blocks are
    reused and overwritten by another request, it is swapped back into other
    GPU blocks, and its decode equals the decode before the swap."""
    rng = np.random.default_rng(41)
    Hq, Hkv, D, bs, NB, HNB = 8, 2, 128, 16, 24, 16
    gpu, cpu = pkv.BlockManager(NB - 1, bs), pkv.BlockManager(HNB, bs)
    kc = np.full((NB, Hkv, bs, D), np.nan, np.float16)
    dk, dv = to_dev(kc), to_dev(kc)
    L = 150
    gpu.allocate(0, L)
    k0 = rng.standard_normal((L, Hkv, D)).astype(np.float16)
    v0 = rng.standard_normal((L, Hkv, D)).astype(np.float16)
    pkv.kv_append(to_dev(k0), to_dev(v0), dk, dv, to_dev(gpu.slots(0, 0, L)))
    q = to_dev(rng.standard_normal((1, Hq, D)).astype(np.float16))
    scale = float(np.float32(1 / np.sqrt(D)))

    def decode(r):
        tab, lens = gpu.build_tables([r], 16, pad_block=NB - 1)
        return to_host(pkv.paged_attention_decode(q, dk, dv, to_dev(tab), to_dev(lens),
                                                  max_seq_len=int(lens[0]), scale=scale))
    before = decode(0)
    hk = _pinned_pool((HNB, Hkv, bs, D), np.zeros((HNB, Hkv, bs, D), np.float16))
    hv = _pinned_pool((HNB, Hkv, bs, D), np.zeros((HNB, Hkv, bs, D), np.float16))
    say("swap out request 0")
    src, dst = gpu.swap_to(cpu, 0)
    pkv.copy_blocks(dk, dv, hk, hv, to_dev(src), to_dev(dst))
    gpu.allocate(1, 200)                       # takes the freed blocks and more
    assert set(src) <= set(gpu.block_table(1))
    junk = rng.standard_normal((200, Hkv, D)).astype(np.float16)
    pkv.kv_append(to_dev(junk), to_dev(junk), dk, dv, to_dev(gpu.slots(1, 0, 200)))
    gpu.free(1)
    say("swap in request 0")
    src2, dst2 = cpu.swap_to(gpu, 0)
    pkv.copy_blocks(hk, hv, dk, dv, to_dev(src2), to_dev(dst2))
    assert list(gpu.block_table(0)) != list(src)
    after = decode(0)
    assert np.array_equal(after.view(np.uint32), before.view(np.uint32))
    # and the decode itself against the oracle over the request's own rows
    tab = np.arange(W.cdiv(L, bs), dtype=np.int32)[None]
    pk = np.zeros((tab.shape[1], Hkv, bs, D), np.float16)
    pv = np.zeros_like(pk)
    okc, ovc = oracle.kv_append(k0, v0, pk, pv, np.arange(L, dtype=np.int32))
    ref = oracle.decode(to_host(q), okc, ovc, tab, np.array([L], np.int32), scale)
    assert max_abs(after, ref) <= TIGHT_DECODE


# ------------------------------------------- multi-step continuous batching
def test_driver_steps_match_dense_attention():
    """The scheduler's plans drive append, prefill and decode step after step
    (chunked prompts, mixed prefill/decode batches, finished requests
    releasing blocks, preemption by recompute in a tight pool).  A request's
    rows are a fixed function of (request, position), so recomputed prompts
    rewrite the same K/V; every step's prefill and decode outputs match the
    oracle over that request's contiguous rows."""
    from paged_kv_cache_407_amd.driver import StepDriver
    Hq, Hkv, D, bs, NB = 4, 2, 64, 16, 16            # 15 usable blocks: 9 preemptions
    max_batch, max_tokens, max_len = 6, 96, 256
    rng = np.random.default_rng(77)
    n_req = 14
    reqs = [(int(rng.integers(1, 150)), int(rng.integers(0, 30))) for _ in range(n_req)]
    tabs = {}
    for r in range(n_req):
        g = np.random.default_rng(1000 + r)
        tabs[r] = tuple(g.standard_normal((max_len,) + sh).astype(np.float16)
                        for sh in ((Hkv, D), (Hkv, D), (Hq, D)))
    bm = pkv.BlockManager(NB - 1, bs)                   # block NB-1: pad canary
    sched = pkv.Scheduler(bm, max_batch, max_tokens, max_len)
    kc = to_dev(np.full((NB, Hkv, bs, D), np.nan, np.float16))
    vc = to_dev(np.full((NB, Hkv, bs, D), np.nan, np.float16))
    scale = float(np.float32(1 / np.sqrt(D)))

    def positions(plan):
        pf = []
        for k, r in enumerate(plan["prefill_ids"]):
            n = int(plan["cu_q_lens"][k + 1] - plan["cu_q_lens"][k])
            L = int(plan["prefill_lens"][k])
            pf.append((int(r), np.arange(L - n, L)))
        dec = [(int(r), int(L) - 1) for r, L in zip(plan["decode_ids"], plan["decode_lens"])]
        return pf, dec

    def rows_fn(plan):
        pf, dec = positions(plan)
        k = [tabs[r][0][p] for r, p in pf] + [tabs[r][0][p][None] for r, p in dec]
        v = [tabs[r][1][p] for r, p in pf] + [tabs[r][1][p][None] for r, p in dec]
        q = [tabs[r][2][p] for r, p in pf] + [tabs[r][2][p][None] for r, p in dec]
        return to_dev(np.concatenate(k)), to_dev(np.concatenate(v)), to_dev(np.concatenate(q))

    drv = StepDriver(sched, kc, vc, Hq, scale, rows_fn, pad_block=NB - 1)

    def dense(r, L):
        nb = W.cdiv(L, bs)
        k = np.zeros((nb * bs, Hkv, D), np.float16)
        v = np.zeros_like(k)
        k[:L], v[:L] = tabs[r][0][:L], tabs[r][1][:L]
        pool = lambda a: a.reshape(nb, bs, Hkv, D).transpose(0, 2, 1, 3).copy()  # noqa
        return pool(k), pool(v), np.arange(nb, dtype=np.int32)[None]

    order = list(range(n_req))
    finished, preempted, worst, steps = 0, 0, 0.0, 0
    while finished < n_req and steps < 2000:
        if steps < n_req:                               # one arrival per step
            r = order[steps]
            sched.add_request(r, *reqs[r])
        plan, out_pf, out_dec = drv.step()
        steps += 1
        finished += len(plan["finished"])
        preempted += len(plan["preempted"])
        if out_pf is None and out_dec is None:
            continue
        torch.cuda.synchronize()
        pf, dec = positions(plan)
        if out_pf is not None:
            got = to_host(out_pf)
            for k, (r, pos) in enumerate(pf):
                L = int(pos[-1]) + 1
                pk, pv, tab = dense(r, L)
                q = tabs[r][2][pos]
                ref = oracle.prefill(q, np.array([0, len(pos)], np.int32), pk, pv, tab,
                                     np.array([L], np.int32), scale)
                lo, hi = int(plan["cu_q_lens"][k]), int(plan["cu_q_lens"][k + 1])
                worst = max(worst, max_abs(got[lo:hi], ref))
        if out_dec is not None:
            got = to_host(out_dec)
            for d, (r, p) in enumerate(dec):
                pk, pv, tab = dense(r, p + 1)
                ref = oracle.decode(tabs[r][2][p][None], pk, pv, tab,
                                    np.array([p + 1], np.int32), scale)
                worst = max(worst, max_abs(got[d:d + 1], ref))
    say(f"driver: {steps} steps, {finished} finished, {preempted} preempted, max-abs {worst:.3g}")
    assert finished == n_req and bm.num_free == NB - 1
    assert preempted > 0                                # the tight pool forced it
    assert worst <= TIGHT_PREFILL
