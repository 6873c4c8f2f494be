// Kernel parameter blocks and launchers (internal to libpkv).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct AppendParams {
  const uint4 *key;      // [T][Hkv][D] fp16, as 16-byte chunks
  const uint4 *value;
  uint4 *k_cache;        // [NB][Hkv][BS][D]
  uint4 *v_cache;
  const int32_t *slots;  // [T]
  int32_t num_tokens, num_kv_heads, chunks_per_row, block_size;
  int64_t num_slots;
};

// Longest batch whose dispatch order travels in the kernel arguments.
constexpr int kMaxOrderSeqs = 256;

struct DecodeParams {
  float *out;                   // [S][Hq][D]
  const _Float16 *q;            // [S][Hq][D]
  const _Float16 *k_cache;      // [NB][Hkv][BS][D]
  const _Float16 *v_cache;
  const int32_t *block_tables;  // [S][MB]
  const int32_t *seq_lens;      // [S]
  float *ws_o;                  // [S][Hq][NP][D]   (split only)
  float *ws_m;                  // [S][Hq][NP]
  float *ws_l;                  // [S][Hq][NP]
  int32_t num_seqs, num_q_heads, num_kv_heads, group;
  int32_t num_blocks, max_blocks_per_seq, max_seq_len;
  int32_t part_tokens, num_parts;
  float scale_log2e;
  // Dispatch order (kernel arguments, read with scalar loads): grid slot i
  // runs sequence order[i] when has_order; results do not depend on it.
  int32_t has_order;
  int16_t order[kMaxOrderSeqs];
};

struct PrefillParams {
  float *out;                   // [Tq][Hq][D]
  const _Float16 *q;            // [Tq][Hq][D]
  const int32_t *cu_q_lens;     // [C+1]
  const _Float16 *k_cache;
  const _Float16 *v_cache;
  const int32_t *block_tables;  // [C][MB]
  const int32_t *seq_lens;      // [C]
  int32_t num_chunks, total_q, num_q_heads, num_kv_heads, group;
  int32_t num_blocks, max_blocks_per_seq, max_seq_len;
  float scale_log2e;
  // Key-range split: a query tile with n key tiles runs in
  // min(num_splits, cdiv(n, split_tiles)) parts; with several parts each
  // writes its unnormalised output, maximum and sum here and
  // prefill_merge_kernel combines them.
  float *ws_o;          // [num_splits][total_q][Hq][D]
  float *ws_m, *ws_l;   // [num_splits][total_q][Hq]
  int32_t num_splits, split_tiles;
};

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream);

struct CopyParams {
  const uint4 *src_k, *src_v;  // [src_num_blocks][chunks_per_block]
  uint4 *dst_k, *dst_v;        // [dst_num_blocks][chunks_per_block]
  const int32_t *src_ids, *dst_ids;  // [count], device-accessible
  int32_t count, src_num_blocks, dst_num_blocks;
  int64_t chunks_per_block;    // num_kv_heads * block_size * head_dim / 8
};
hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t stream);
// D in {64,128}, BS in {1,8,16,32}; returns hipErrorInvalidValue otherwise.
// part_tokens must be a multiple of BS and at most max_partition_blocks() *
// BS: a wave keeps a partition's block ids kIdsPerLane per lane (256
// blocks), or one per lane (64 blocks) when blocks are smaller than a
// wave-wide load and each lane fetches its own token's id by a lane permute
// (block size 1).
constexpr int kMaxPartBlocks = 64;
constexpr int kIdsPerLane = 4;
constexpr int kMaxPartBlocksWide = 64 * kIdsPerLane;
// Query heads one decode workgroup serves: the largest of 8, 4, 2, 1 that
// divides the group of query heads sharing one KV head, or 16 when 16
// divides it and the matrix-core kernel serves the block size (>= 8).
inline int heads_per_workgroup(int group, int block_size) {
  if (group % 16 == 0 && block_size >= 8) return 16;
  return group % 8 == 0 ? 8 : group % 4 == 0 ? 4 : group % 2 == 0 ? 2 : 1;
}
// The decode runs on the matrix cores when a workgroup serves 4 or more
// query heads and a 16-row tile lies in one or two blocks.
inline bool decode_on_mfma(int group, int block_size) {
  return heads_per_workgroup(group, block_size) >= 4 && block_size >= 8;
}
inline int max_partition_blocks(int block_size) {
  return block_size >= 8 ? kMaxPartBlocksWide : kMaxPartBlocks;
}
hipError_t launch_decode(const DecodeParams &p, int head_dim, int block_size,
                         hipStream_t stream);
hipError_t launch_prefill(const PrefillParams &p, int head_dim,
                          int block_size, int max_q_len, hipStream_t stream);

}  // namespace pkv
