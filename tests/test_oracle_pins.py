"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import pins
import workloads as W


@pytest.mark.parametrize("name", pins.ALL_PINS)
def test_pin(orc, name):
    pins.run_pin(orc, name)


@pytest.mark.parametrize("spec", pins.small_specs(), ids=lambda s: s.name)
def test_dense_decode_small(orc, spec):
    pins.pin_dense_decode(orc, spec)


def test_dense_decode_tiny_config(orc):
    # the tiny workload exactly as benchmarked
    pins.pin_dense_decode(orc, W.SPECS["tiny"])


@pytest.mark.parametrize("name", ["llama_decode", "mixed", "gqa_shared", "long"])
def test_dense_equivalence_at_config_scale(orc, name):
    # the paged oracle on sampled rows of the benchmark batches (their real
    # pools, tables and lengths, including the shared prefix and 32K
    # contexts) against float64 attention over the contiguous K/V
    err = pins.pin_dense_config(orc, name)
    print(f"{name}: oracle vs dense float64 attention {err:.3g}")


def test_oracle_rejects_bad_input(orc):
    import oracle
    b = W.make_batch("tiny")
    slots = b.slot_mapping.copy()
    slots[1] = slots[0]
    with pytest.raises(oracle.OracleError, match="duplicate"):
        orc.kv_append(b.new_k, b.new_v, b.k_cache, b.v_cache, slots)
    slots = b.slot_mapping.copy()
    slots[0] = b.spec.num_blocks * b.spec.block_size
    with pytest.raises(oracle.OracleError, match="range"):
        orc.kv_append(b.new_k, b.new_v, b.k_cache, b.v_cache, slots)
    tab = b.tables_dec.copy()
    tab[0, 0] = b.spec.num_blocks
    with pytest.raises(oracle.OracleError, match="range"):
        orc.decode(b.q_dec, b.k_cache, b.v_cache, tab, b.lens_dec, b.scale)
    lens = b.lens_dec.copy()
    lens[0] = 0
    with pytest.raises(oracle.OracleError, match="bad argument"):
        orc.decode(b.q_dec, b.k_cache, b.v_cache, b.tables_dec, lens, b.scale)


def test_rows_subset_matches_full(orc):
    b = W.make_batch("tiny")
    kc, vc = pins.appended(orc, b)
    full = orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale)
    rows = [0, 5, 15]
    part = orc.decode(b.q_dec, kc, vc, b.tables_dec, b.lens_dec, b.scale, rows=rows)
    flat_f = full.reshape(-1, full.shape[-1])
    flat_p = part.reshape(-1, part.shape[-1])
    assert np.array_equal(flat_f[rows], flat_p[rows])
    assert np.isnan(np.delete(flat_p, rows, axis=0)).all()


def test_kv_bytes_per_token_matches_page():
    g = pins.golden("kv_bytes.json")
    per = W.kv_bytes_per_token(g["num_layers"], g["num_kv_heads"], g["head_dim"],
                               g["elem_bytes"])
    assert per == g["bytes_per_token"]
    assert per * g["tokens"] == g["bytes_for_tokens"]
