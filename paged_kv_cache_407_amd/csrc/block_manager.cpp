// Host-side KV block manager: the free list and per-request block tables
// that produce the block tables and slot mappings the kernels consume.
//
// It follows the block manager of "LLM 推理引擎 Continuous Batching 与
// PagedAttention：从 vLLM 原理到生产级部署实战", §3.2:
// * the free list starts as the block ids 0 .. N-1 and blocks are taken from
//   its end, freed blocks are appended to it (so the last one freed is the
//   first one reused);
// * a request of n tokens takes ceil(n / block_size) blocks, or nothing at
//   all when the free list is too short (out of memory);
// * a new token goes into the request's last block while that block has
//   room, otherwise into a newly taken block;
// * freeing returns a request's blocks to the free list.
// Shared prefixes (same page, §4.1) are whole blocks referenced by several
// tables, with a reference count deciding when a block goes back to the
// free list.  Only full blocks are shared, and a request never appends into
// a full block, so a shared block is never written after it is shared.
//
// Swapping (same page, §4.4) pairs two managers, one over the device pool
// and one over a host pool: moving a request from one to the other takes
// blocks for its tokens in the target, releases its blocks in the source and
// reports the (source, target) block pairs for the copy.
//
// Plain host code (no device calls), not thread-safe.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int32_t len = 0;  // tokens held
  };
  int32_t num_blocks, block_size;
  std::vector<int32_t> free_list;  // taken from the back
  std::vector<int32_t> refs;       // tables referencing each block
  std::unordered_map<int64_t, Seq> seqs;

  pkv_block_manager(int32_t nb, int32_t bs)
      : num_blocks(nb), block_size(bs), refs(nb, 0) {
    free_list.reserve(nb);
    for (int32_t b = 0; b < nb; ++b) free_list.push_back(b);
  }
  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    refs[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refs[b] == 0) free_list.push_back(b);
  }
  Seq *find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
};

extern "C" {

pkv_block_manager *pkv_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  return new (std::nothrow) pkv_block_manager(num_blocks, block_size);
}

void pkv_bm_destroy(pkv_block_manager *bm) { delete bm; }

int32_t pkv_bm_num_free(const pkv_block_manager *bm) {
  return bm ? (int32_t)bm->free_list.size() : -1;
}

int32_t pkv_bm_block_size(const pkv_block_manager *bm) {
  return bm ? bm->block_size : -1;
}

int pkv_bm_allocate(pkv_block_manager *bm, int64_t request_id,
                    int32_t num_tokens) {
  if (!bm || num_tokens < 0 || bm->find(request_id)) return PKV_ERR_INVALID;
  const int64_t need = ((int64_t)num_tokens + bm->block_size - 1) / bm->block_size;
  if ((int64_t)bm->free_list.size() < need) return PKV_ERR_NO_BLOCKS;
  pkv_block_manager::Seq s;
  s.len = num_tokens;
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  bm->seqs.emplace(request_id, std::move(s));
  return PKV_OK;
}

int pkv_bm_append_token(pkv_block_manager *bm, int64_t request_id,
                        int32_t *slot) {
  if (!bm || !slot) return PKV_ERR_INVALID;
  pkv_block_manager::Seq *s = bm->find(request_id);
  if (!s) return PKV_ERR_INVALID;
  const int32_t pos = s->len;
  if (pos % bm->block_size == 0) {  // the last block is full (or none yet)
    if (bm->free_list.empty()) return PKV_ERR_NO_BLOCKS;
    s->blocks.push_back(bm->take());
  }
  *slot = s->blocks[pos / bm->block_size] * bm->block_size + pos % bm->block_size;
  s->len = pos + 1;
  return PKV_OK;
}

int pkv_bm_append_tokens(pkv_block_manager *bm, const int64_t *request_ids,
                         int32_t count, int32_t *slots) {
  if (!bm || count < 0 || (count && (!request_ids || !slots)))
    return PKV_ERR_INVALID;
  // all or nothing: check ids, duplicates and the blocks needed first
  int64_t need = 0;
  std::unordered_map<int64_t, int32_t> seen;
  for (int32_t i = 0; i < count; ++i) {
    const pkv_block_manager::Seq *s = bm->find(request_ids[i]);
    if (!s || seen.count(request_ids[i])) return PKV_ERR_INVALID;
    seen[request_ids[i]] = 1;
    if (s->len % bm->block_size == 0) ++need;
  }
  if ((int64_t)bm->free_list.size() < need) return PKV_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < count; ++i)
    pkv_bm_append_token(bm, request_ids[i], &slots[i]);
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager *bm, int64_t parent_id, int64_t child_id,
                int32_t prefix_tokens) {
  if (!bm || parent_id == child_id || bm->find(child_id)) return PKV_ERR_INVALID;
  const pkv_block_manager::Seq *p = bm->find(parent_id);
  if (!p || prefix_tokens < 0 || prefix_tokens > p->len) return PKV_ERR_INVALID;
  pkv_block_manager::Seq c;
  const int32_t full = prefix_tokens / bm->block_size;
  for (int32_t i = 0; i < full; ++i) {
    c.blocks.push_back(p->blocks[i]);
    ++bm->refs[p->blocks[i]];
  }
  c.len = full * bm->block_size;
  bm->seqs.emplace(child_id, std::move(c));
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager *bm, int64_t request_id) {
  if (!bm) return PKV_ERR_INVALID;
  auto it = bm->seqs.find(request_id);
  if (it == bm->seqs.end()) return PKV_ERR_INVALID;
  for (int32_t b : it->second.blocks) bm->release(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

int32_t pkv_bm_seq_len(const pkv_block_manager *bm, int64_t request_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(request_id);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_bm_block_table(const pkv_block_manager *bm, int64_t request_id,
                           int32_t *blocks, int32_t capacity) {
  if (!bm || capacity < 0) return -1;
  auto it = bm->seqs.find(request_id);
  if (it == bm->seqs.end()) return -1;
  const int32_t n = (int32_t)it->second.blocks.size();
  for (int32_t i = 0; i < n && i < capacity; ++i) blocks[i] = it->second.blocks[i];
  return n;
}

int pkv_bm_build_tables(const pkv_block_manager *bm, const int64_t *request_ids,
                        int32_t count, int32_t max_blocks_per_seq,
                        int32_t pad_block, int32_t *block_tables,
                        int32_t *seq_lens) {
  if (!bm || count < 0 || max_blocks_per_seq <= 0 ||
      (count && (!request_ids || !block_tables || !seq_lens)))
    return PKV_ERR_INVALID;
  for (int32_t i = 0; i < count; ++i) {
    auto it = bm->seqs.find(request_ids[i]);
    if (it == bm->seqs.end() ||
        (int32_t)it->second.blocks.size() > max_blocks_per_seq)
      return PKV_ERR_INVALID;
    int32_t *row = block_tables + (int64_t)i * max_blocks_per_seq;
    const std::vector<int32_t> &b = it->second.blocks;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int32_t)b.size() ? b[j] : pad_block;
    seq_lens[i] = it->second.len;
  }
  return PKV_OK;
}

int pkv_bm_slots(const pkv_block_manager *bm, int64_t request_id,
                 int32_t first_pos, int32_t count, int32_t *slots) {
  if (!bm || first_pos < 0 || count < 0 || (count && !slots))
    return PKV_ERR_INVALID;
  auto it = bm->seqs.find(request_id);
  if (it == bm->seqs.end() || (int64_t)first_pos + count > it->second.len)
    return PKV_ERR_INVALID;
  const int32_t bs = bm->block_size;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t p = first_pos + i;
    slots[i] = it->second.blocks[p / bs] * bs + p % bs;
  }
  return PKV_OK;
}

int pkv_bm_swap(pkv_block_manager *from, pkv_block_manager *to, int64_t request_id,
                int32_t *src_blocks, int32_t *dst_blocks, int32_t capacity,
                int32_t *count) {
  if (!from || !to || from == to || !count || capacity < 0 ||
      from->block_size != to->block_size)
    return PKV_ERR_INVALID;
  auto it = from->seqs.find(request_id);
  if (it == from->seqs.end() || to->find(request_id)) return PKV_ERR_INVALID;
  const std::vector<int32_t> &held = it->second.blocks;
  const int32_t n = (int32_t)held.size();
  if (n > capacity || (n && (!src_blocks || !dst_blocks))) return PKV_ERR_INVALID;
  if ((int32_t)to->free_list.size() < n) return PKV_ERR_NO_BLOCKS;
  pkv_block_manager::Seq moved;
  moved.len = it->second.len;
  for (int32_t i = 0; i < n; ++i) {
    moved.blocks.push_back(to->take());
    src_blocks[i] = held[i];
    dst_blocks[i] = moved.blocks[i];
  }
  to->seqs.emplace(request_id, std::move(moved));
  for (int32_t b : held) from->release(b);  // shared blocks stay with their other owners
  from->seqs.erase(it);
  *count = n;
  return PKV_OK;
}

}  // extern "C"
