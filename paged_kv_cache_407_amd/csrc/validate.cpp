// Host-side checks of the preconditions that the kernels cannot verify
// without a synchronisation: the device copies of these arrays are read by
// the kernels, which only guard against out-of-pool reads (NaN rows, skipped
// slots).  A caller that keeps a host copy of a step's arrays -- the block
// manager and the scheduler write them on the host -- can check it here
// before the copy to the device.
//
// The conditions follow the cache layout of "LLM 推理引擎 Continuous
// Batching 与 PagedAttention：从 vLLM 原理到生产级部署实战":
// * §3.2 (append_token): a new token's place is block slot / block_size,
//   offset slot % block_size; one token per place;
// * §3.3 (the kernel's table lookup): logical block t / block_size of
//   sequence s is block_tables[s][t / block_size], which must name a
//   physical block of the pool for every token below seq_len;
// * §4.3 (chunked prefill): a chunk of C new tokens ends its sequence, so
//   0 <= C <= seq_len, and the chunks' rows are packed in order.
//
// Plain host code; no device calls.  The status strings of the whole
// library live here too (host code, also in the host-only builds).
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "pkv.h"

namespace {

int fail(int64_t *bad_index, int64_t i) {
  if (bad_index) *bad_index = i;
  return PKV_ERR_INVALID;
}

int pass(int64_t *bad_index) {
  if (bad_index) *bad_index = -1;
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_validate_slots(const int32_t *slot_mapping, int32_t num_tokens, int32_t num_blocks,
                       int32_t block_size, int64_t *bad_index) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 ||
      (num_tokens > 0 && !slot_mapping))
    return fail(bad_index, -1);
  const int64_t places = (int64_t)num_blocks * block_size;
  std::vector<int64_t> order;
  order.reserve(num_tokens);
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t slot = slot_mapping[i];
    if (slot < 0) continue;  // padding row
    if (slot >= places) return fail(bad_index, i);
    order.push_back((int64_t)slot << 32 | (uint32_t)i);
  }
  // the first row whose slot an earlier row already holds
  std::sort(order.begin(), order.end());
  int64_t first_dup = -1;
  for (size_t k = 1; k < order.size(); ++k)
    if ((order[k] >> 32) == (order[k - 1] >> 32)) {
      const int64_t row = order[k] & 0xffffffff;
      if (first_dup < 0 || row < first_dup) first_dup = row;
    }
  if (first_dup >= 0) return fail(bad_index, first_dup);
  return pass(bad_index);
}

int pkv_validate_tables(const int32_t *block_tables, const int32_t *seq_lens,
                        int32_t num_seqs, int32_t max_blocks_per_seq, int32_t num_blocks,
                        int32_t block_size, int64_t *bad_index) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0 ||
      (num_seqs > 0 && (!block_tables || !seq_lens)))
    return fail(bad_index, -1);
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = seq_lens[s];
    if (L < 1 || L > cap) return fail(bad_index, (int64_t)s * max_blocks_per_seq);
    const int32_t live = (int32_t)((L + (int64_t)block_size - 1) / block_size);
    const int32_t *row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int32_t j = 0; j < live; ++j)
      if (row[j] < 0 || row[j] >= num_blocks)
        return fail(bad_index, (int64_t)s * max_blocks_per_seq + j);
  }
  return pass(bad_index);
}

int pkv_validate_chunks(const int32_t *cu_q_lens, const int32_t *seq_lens, int32_t num_chunks,
                        int32_t total_q_tokens, int64_t *bad_index) {
  if (num_chunks < 0 || total_q_tokens < 0 || !cu_q_lens ||
      (num_chunks > 0 && !seq_lens))
    return fail(bad_index, -1);
  if (cu_q_lens[0] != 0) return fail(bad_index, 0);
  for (int32_t c = 0; c < num_chunks; ++c) {
    const int32_t len = cu_q_lens[c + 1] - cu_q_lens[c];
    if (len < 0 || len > seq_lens[c] || cu_q_lens[c + 1] > total_q_tokens)
      return fail(bad_index, c);
  }
  if (cu_q_lens[num_chunks] != total_q_tokens) return fail(bad_index, num_chunks);
  return pass(bad_index);
}

const char *pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape (head_dim 64/128; block_size 1/8/16/32 for decode, 8/16/32 for prefill)";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_NO_BLOCKS: return "not enough free KV blocks";
    case PKV_ERR_SCRATCH:
      return "the call's split partials exceed the no-allocation decode's device scratch "
             "(PKV_NOALLOC_SCRATCH_BYTES); pass a workspace to pkv_paged_attention_decode";
    default: return "unknown status";
  }
}

}  // extern "C"
