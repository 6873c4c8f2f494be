/*
 * CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg load this library.  The GPU product path never calls it and shares no
 * source with it.
 *
 * It is the plain definition of what the paged-attention hot path computes,
 * written for a reader to check by eye, in double precision on the fp16 bit
 * patterns it is given:
 *
 *   kv append   -- a new token whose slot is `slot` lands in physical block
 *                  slot / block_size at offset slot % block_size
 *                  ("LLM 推理引擎 Continuous Batching 与 PagedAttention：从 vLLM
 *                  原理到生产级部署实战", §3.2 BlockManager.append_token);
 *   gather      -- logical token t of a sequence is read from physical block
 *                  block_tables[seq][t / block_size] at offset t % block_size,
 *                  and only the first seq_len tokens exist (same page, §3.3,
 *                  the kernel's block-table lookup and tokens_in_block bound);
 *   attention   -- scores q.k_t * scale, softmax over the sequence's tokens,
 *                  output sum_t softmax_t * v_t.  The page's kernel stops after
 *                  the running max/sum and leaves the V weighting out; this
 *                  takes the plain reading: divide by the sum of exponentials
 *                  and weight V (same page, §3.3, closing comment).
 *   prefill     -- query row j of a chunk that sits on a cached prefix of P
 *                  tokens has absolute position P + j and sees keys 0..P+j
 *                  (same page, §4.3 Chunked Prefill; the causal rule of the
 *                  prefill phase in §1.1).
 *   block copy  -- swapping moves a request's KV from its GPU blocks to CPU
 *                  blocks and back (same page, §4.4 Swap): every element of
 *                  a source block, all KV heads and positions, K and V, is
 *                  copied to the paired destination block.
 *
 * Softmax is computed in two passes (maximum first, then exponentials),
 * deliberately not with the GPU's running-max recurrence.
 *
 * Layouts (all row-major):
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim] fp16
 *   q (decode)       : [num_seqs][num_q_heads][head_dim] fp16
 *   q (prefill)      : [total_q][num_q_heads][head_dim] fp16, chunk c's rows
 *                      are cu_q_lens[c] .. cu_q_lens[c+1]-1
 *   block_tables     : [num_seqs][max_blocks_per_seq] int32
 *   out              : same row layout as q, double
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Return codes: 0 ok; 1 bad argument; 2 a slot or block id out of range;
 * 3 duplicate slot; 4 out of memory.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads of the OpenMP loops below (for timing the oracle on one core);
 * n <= 0 restores the count the process started with.  Not arithmetic. */
void oracle_set_threads(int n)
{
    static int initial = 0;
    if (!initial)
        initial = omp_get_max_threads();
    omp_set_num_threads(n > 0 ? n : initial);
}

/* IEEE 754 binary16 -> double, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 encodes zero and
 * subnormals (fraction * 2^-24), exponent 31 encodes infinities and NaNs. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac | 0x400), expo - 25);
    return sign ? -v : v;
}

/* Writes each new row into its slot.  Rows with a negative slot are skipped.
 * key, value: [num_tokens][num_kv_heads][head_dim] fp16 bits. */
int oracle_kv_append(const uint16_t *key, const uint16_t *value,
                     uint16_t *k_cache, uint16_t *v_cache,
                     const int32_t *slot_mapping, int32_t num_tokens,
                     int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks)
{
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks <= 0)
        return 1;
    int64_t nslots = (int64_t)num_blocks * block_size;
    /* Each slot may be written by at most one row. */
    unsigned char *seen = calloc((size_t)nslots, 1);
    if (!seen)
        return 4;
    for (int32_t i = 0; i < num_tokens; i++) {
        int32_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        if (slot >= nslots) {
            free(seen);
            return 2;
        }
        if (seen[slot]) {
            free(seen);
            return 3;
        }
        seen[slot] = 1;
    }
    free(seen);

    for (int32_t i = 0; i < num_tokens; i++) {
        int32_t slot = slot_mapping[i];
        if (slot < 0)
            continue;
        int64_t blk = slot / block_size;
        int64_t off = slot % block_size;
        for (int32_t h = 0; h < num_kv_heads; h++) {
            for (int32_t d = 0; d < head_dim; d++) {
                int64_t src = ((int64_t)i * num_kv_heads + h) * head_dim + d;
                int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * head_dim + d;
                k_cache[dst] = key[src];
                v_cache[dst] = value[src];
            }
        }
    }
    return 0;
}

/* For i < count: block src_blocks[i] of (src_k, src_v) -> block dst_blocks[i]
 * of (dst_k, dst_v), element by element.  Pools [nb][num_kv_heads]
 * [block_size][head_dim] fp16 bits.  An id outside its pool is an error (2),
 * a destination named twice is an error (3). */
int oracle_copy_blocks(const uint16_t *src_k, const uint16_t *src_v,
                       uint16_t *dst_k, uint16_t *dst_v,
                       const int32_t *src_blocks, const int32_t *dst_blocks,
                       int32_t count, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t src_num_blocks,
                       int32_t dst_num_blocks)
{
    if (count < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        src_num_blocks <= 0 || dst_num_blocks <= 0)
        return 1;
    unsigned char *seen = calloc((size_t)dst_num_blocks, 1);
    if (!seen)
        return 4;
    for (int32_t i = 0; i < count; i++) {
        int32_t s = src_blocks[i], d = dst_blocks[i];
        if (s < 0 || s >= src_num_blocks || d < 0 || d >= dst_num_blocks) {
            free(seen);
            return 2;
        }
        if (seen[d]) {
            free(seen);
            return 3;
        }
        seen[d] = 1;
    }
    free(seen);
    for (int32_t i = 0; i < count; i++) {
        int64_t s = src_blocks[i], d = dst_blocks[i];
        for (int32_t h = 0; h < num_kv_heads; h++)
            for (int32_t o = 0; o < block_size; o++)
                for (int32_t e = 0; e < head_dim; e++) {
                    int64_t from = ((s * num_kv_heads + h) * block_size + o) * head_dim + e;
                    int64_t to = ((d * num_kv_heads + h) * block_size + o) * head_dim + e;
                    dst_k[to] = src_k[from];
                    dst_v[to] = src_v[from];
                }
    }
    return 0;
}

/* Attention of one query row against the first n_keys logical tokens of the
 * sequence whose block-table row is `table`, KV head kvh.  Writes head_dim
 * doubles to out.  scores: scratch of n_keys doubles. */
static int attend(double *out, const uint16_t *qrow, const uint16_t *k_cache,
                  const uint16_t *v_cache, const int32_t *table,
                  int32_t n_keys, int32_t kvh, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                  double scale, double *scores)
{
    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (int32_t t = 0; t < n_keys; t++) {
        int32_t phys = table[t / block_size];
        if (phys < 0 || phys >= num_blocks)
            return 2;
        const uint16_t *k = k_cache +
            (((int64_t)phys * num_kv_heads + kvh) * block_size + t % block_size) * head_dim;
        double dot = 0.0;
        for (int32_t d = 0; d < head_dim; d++)
            dot += oracle_half_to_double(qrow[d]) * oracle_half_to_double(k[d]);
        scores[t] = dot * scale;
        if (scores[t] > m)
            m = scores[t];
    }
    /* pass 2: exponentials, their sum, and the weighted sum of values */
    double l = 0.0;
    for (int32_t d = 0; d < head_dim; d++)
        out[d] = 0.0;
    for (int32_t t = 0; t < n_keys; t++) {
        double e = exp(scores[t] - m);
        l += e;
        int32_t phys = table[t / block_size];
        const uint16_t *v = v_cache +
            (((int64_t)phys * num_kv_heads + kvh) * block_size + t % block_size) * head_dim;
        for (int32_t d = 0; d < head_dim; d++)
            out[d] += e * oracle_half_to_double(v[d]);
    }
    for (int32_t d = 0; d < head_dim; d++)
        out[d] /= l;
    return 0;
}

static int check_shapes(int32_t nq, int32_t hq, int32_t hkv, int32_t d,
                        int32_t bs, int32_t nb, int32_t mb)
{
    if (nq < 0 || hq <= 0 || hkv <= 0 || d <= 0 || bs <= 0 || nb <= 0 || mb <= 0)
        return 1;
    if (hq % hkv)
        return 1;
    return 0;
}

/* Decode: one query token per sequence attends to all seq_lens[s] tokens.
 * rows: optional list of (s * num_q_heads + h) row ids to compute (NULL =
 * all); only those rows of out are written. */
int oracle_decode(double *out, const uint16_t *q, const uint16_t *k_cache,
                  const uint16_t *v_cache, const int32_t *block_tables,
                  int32_t max_blocks_per_seq, const int32_t *seq_lens,
                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                  double scale, const int64_t *rows, int64_t num_rows)
{
    if (check_shapes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq))
        return 1;
    for (int32_t s = 0; s < num_seqs; s++)
        if (seq_lens[s] < 1 || seq_lens[s] > (int64_t)max_blocks_per_seq * block_size)
            return 1;
    int64_t n = rows ? num_rows : (int64_t)num_seqs * num_q_heads;
    int32_t group = num_q_heads / num_kv_heads;
    int status = 0;
#pragma omp parallel
    {
        int32_t maxlen = (int32_t)max_blocks_per_seq * block_size;
        double *scores = malloc(sizeof(double) * (size_t)maxlen);
        if (!scores) {
#pragma omp atomic write
            status = 4;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; i++) {
            if (!scores)
                continue;
            int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= (int64_t)num_seqs * num_q_heads) {
#pragma omp atomic write
                status = 1;
                continue;
            }
            int32_t s = (int32_t)(r / num_q_heads), h = (int32_t)(r % num_q_heads);
            int rc = attend(out + r * head_dim, q + r * head_dim, k_cache, v_cache,
                            block_tables + (int64_t)s * max_blocks_per_seq,
                            seq_lens[s], h / group, num_kv_heads, head_dim,
                            block_size, num_blocks, scale, scores);
            if (rc) {
#pragma omp atomic write
                status = rc;
            }
        }
        free(scores);
    }
    return status;
}

/* Prefill: chunk c owns query rows cu_q_lens[c] .. cu_q_lens[c+1]-1, and its
 * sequence holds seq_lens[c] tokens after this chunk was appended, so the
 * chunk's cached prefix is P = seq_lens[c] - chunk length.  Row j attends to
 * keys 0 .. P + j.  rows: optional list of (token * num_q_heads + h). */
int oracle_prefill(double *out, const uint16_t *q, const int32_t *cu_q_lens,
                   const uint16_t *k_cache, const uint16_t *v_cache,
                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *seq_lens, int32_t num_chunks,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t num_blocks, double scale,
                   const int64_t *rows, int64_t num_rows)
{
    if (check_shapes(num_chunks, num_q_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq))
        return 1;
    if (cu_q_lens[0] != 0)
        return 1;
    for (int32_t c = 0; c < num_chunks; c++) {
        int32_t len = cu_q_lens[c + 1] - cu_q_lens[c];
        if (len < 0 || len > seq_lens[c] || seq_lens[c] < 1 ||
            seq_lens[c] > (int64_t)max_blocks_per_seq * block_size)
            return 1;
    }
    int64_t total = cu_q_lens[num_chunks];
    int64_t n = rows ? num_rows : total * num_q_heads;
    int32_t group = num_q_heads / num_kv_heads;
    int status = 0;
#pragma omp parallel
    {
        int32_t maxlen = (int32_t)max_blocks_per_seq * block_size;
        double *scores = malloc(sizeof(double) * (size_t)maxlen);
        if (!scores) {
#pragma omp atomic write
            status = 4;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; i++) {
            if (!scores)
                continue;
            int64_t r = rows ? rows[i] : i;
            if (r < 0 || r >= total * num_q_heads) {
#pragma omp atomic write
                status = 1;
                continue;
            }
            int64_t tok = r / num_q_heads;
            int32_t h = (int32_t)(r % num_q_heads);
            int32_t c = 0;
            while (cu_q_lens[c + 1] <= tok)
                c++;
            int32_t j = (int32_t)(tok - cu_q_lens[c]);
            int32_t prefix = seq_lens[c] - (cu_q_lens[c + 1] - cu_q_lens[c]);
            int rc = attend(out + r * head_dim, q + r * head_dim, k_cache, v_cache,
                            block_tables + (int64_t)c * max_blocks_per_seq,
                            prefix + j + 1, h / group, num_kv_heads, head_dim,
                            block_size, num_blocks, scale, scores);
            if (rc) {
#pragma omp atomic write
                status = rc;
            }
        }
        free(scores);
    }
    return status;
}
