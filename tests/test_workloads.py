"""The seeded input generator: determinism, shapes and canaries (CPU)."""
import numpy as np
import pytest

import workloads as W


def test_deterministic_and_seeded():
    a = W.make_batch("tiny", pad_rows=2)
    b = W.make_batch("tiny", pad_rows=2, threads=1)
    for f in ("k_cache", "v_cache", "new_k", "new_v", "slot_mapping", "q_dec",
              "tables_dec", "lens_dec"):
        x, y = getattr(a, f), getattr(b, f)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f
    c = W.make_batch("tiny", seed=1)
    assert not np.array_equal(a.q_dec, c.q_dec)


def test_tiny_layout():
    b = W.make_batch("tiny", pad_rows=3)
    assert list(b.lens_dec) == [5, 16, 17, 40]
    assert b.k_cache.shape == (64, 4, 16, 64)
    assert (b.slot_mapping == -1).sum() == 3
    assert b.new_k.shape == (4 + 3, 4, 64)
    # canary block is NaN throughout and fills every unused table entry
    assert np.isnan(b.k_cache[b.canary_block]).all()
    live = sum(W.cdiv(int(L), 16) for L in b.lens_dec)
    assert live == 7
    for s, L in enumerate(b.lens_dec):
        n = W.cdiv(int(L), 16)
        assert (b.tables_dec[s, n:] == b.canary_block).all()
        assert len(set(b.tables_dec[s, :n].tolist())) == n
    # the slot of the new token is a NaN canary before the append
    for slot in b.slot_mapping[b.slot_mapping >= 0]:
        blk, off = divmod(int(slot), 16)
        assert np.isnan(b.k_cache[blk, :, off]).all()
    assert W.decode_kv_bytes(b)["logical"] == 78 * 4 * 64 * 2 * 2


def test_mixed_shapes():
    b = W.make_batch("mixed")
    assert b.num_pf == 4 and b.num_dec == 60
    assert b.new_k.shape[0] == 4 * 512 + 60
    assert (b.lens_pf - 512 >= 0).all() and (b.lens_pf <= 1024).all()
    assert (b.lens_dec >= 64).all() and (b.lens_dec <= 2048).all()
    assert list(b.cu_q_lens) == [0, 512, 1024, 1536, 2048]
    assert len(np.unique(b.slot_mapping)) == b.slot_mapping.size
    assert W.prefill_flops(b) > 0


def test_gqa_shared_prefix():
    b = W.make_batch("gqa_shared")
    assert (b.lens_dec >= 256).all() and (b.lens_dec <= 4096).all()
    sh = b.extra["shared_blocks"]
    assert sh.size == 16
    for s, L in enumerate(b.lens_dec):
        n_sh = min(16, (int(L) - 1) // 32)
        assert np.array_equal(b.tables_dec[s, :n_sh], sh[:n_sh])
        assert not np.isin(b.tables_dec[s, n_sh:W.cdiv(int(L), 32)], sh).any()
    by = W.decode_kv_bytes(b)
    assert by["unique"] < by["logical"]
    assert len(np.unique(b.slot_mapping)) == b.slot_mapping.size


def test_llama_decode_shapes():
    b = W.make_batch("llama_decode")
    assert b.num_dec == 32 and b.tables_dec.shape == (32, 64)
    assert (b.lens_dec >= 64).all() and (b.lens_dec <= 1024).all()
    assert b.new_k.shape == (32, 32, 128)
