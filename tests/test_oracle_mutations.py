"""Plants plausible mistakes in copies of the oracle's C source (on the CPU)
and checks that each one fails at least one pin.  This shows that the pins
constrain every step the oracle takes: decoding fp16, the slot arithmetic of
the append, the block-table gather, the head mapping, the scale, the softmax
and its normalisation, and the causal bound of a chunk on a prefix."""
import subprocess

import pytest

import oracle
import pins

MUTATIONS = [
    ("subnormal exponent", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("exponent bias", "expo - 25)", "expo - 24)"),
    ("append offset", "int64_t off = slot % block_size;", "int64_t off = slot % (block_size + 1) % block_size;"),
    ("append block", "int64_t blk = slot / block_size;", "int64_t blk = slot / block_size / 2;"),
    ("append layout", "int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim + d;",
     "int64_t dst = ((blk * block_size + off) * num_kv_heads + h) * head_dim + d;"),
    ("append value", "v_cache[dst] = value[src];", "v_cache[dst] = key[src];"),
    ("gather offset (K)",
     "(((int64_t)phys * num_kv_heads + kvh) * block_size + t % block_size) * head_dim;\n        double dot",
     "(((int64_t)phys * num_kv_heads + kvh) * block_size + (t + 1) % block_size) * head_dim;\n        double dot"),
    ("gather layout (K)",
     "(((int64_t)phys * num_kv_heads + kvh) * block_size + t % block_size) * head_dim;\n        double dot",
     "(((int64_t)phys * block_size + t % block_size) * num_kv_heads + kvh) * head_dim;\n        double dot"),
    ("table row", "int32_t phys = table[t / block_size];\n        if",
     "int32_t phys = table[(t + 1) / block_size];\n        if"),
    ("V read from K", "const uint16_t *v = v_cache +", "const uint16_t *v = k_cache +"),
    ("scale dropped", "scores[t] = dot * scale;", "scores[t] = dot;"),
    ("softmax sign", "double e = exp(scores[t] - m);", "double e = exp(m - scores[t]);"),
    ("no normalisation", "out[d] /= l;", "out[d] /= 1.0;"),
    ("kv head mapping (decode)", "seq_lens[s], h / group,", "seq_lens[s], h % num_kv_heads,"),
    ("table stride", "block_tables + (int64_t)s * max_blocks_per_seq,",
     "block_tables + (int64_t)s * (max_blocks_per_seq - 1),"),
    ("causal bound", "prefix + j + 1, h / group", "prefix + j, h / group"),
    ("chunk prefix", "int32_t prefix = seq_lens[c] - (cu_q_lens[c + 1] - cu_q_lens[c]);",
     "int32_t prefix = seq_lens[c] - (cu_q_lens[c + 1] - cu_q_lens[c]) - 1;"),
    ("last token dropped", "seq_lens[s], h / group,", "seq_lens[s] - (seq_lens[s] > 1), h / group,"),
    ("copy layout", "int64_t to = ((d * num_kv_heads + h) * block_size + o) * head_dim + e;",
     "int64_t to = ((d * block_size + o) * num_kv_heads + h) * head_dim + e;"),
    ("copy V from K", "dst_v[to] = src_v[from];", "dst_v[to] = src_k[from];"),
    ("copy wrong pair", "int64_t s = src_blocks[i], d = dst_blocks[i];",
     "int64_t s = src_blocks[(i + 1) % count], d = dst_blocks[i];"),
    ("copy offset", "int64_t from = ((s * num_kv_heads + h) * block_size + o) * head_dim + e;",
     "int64_t from = ((s * num_kv_heads + h) * block_size + (block_size - 1 - o)) * head_dim + e;"),
]


@pytest.fixture(scope="module")
def source():
    return oracle.SOURCE_PATH.read_text()


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, source, desc, old, new):
    assert source.count(old) == 1, f"mutation anchor not unique: {desc}"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-o", str(lib), str(src), "-lm"], check=True)
    mutant = oracle.Oracle(lib)
    failed = []
    for name in pins.ALL_PINS:
        try:
            pins.run_pin(mutant, name)
        except (AssertionError, oracle.OracleError) as e:
            failed.append((name, str(e)[:80]))
    assert failed, f"no pin catches the planted mistake: {desc}"
