// C ABI of libpkv: argument checks, split choice and kernel launches.
// The functions and their contracts are declared in include/pkv.h.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"
#include "pkv.h"

using namespace pkv;

namespace {

// Default split: the largest partition (4096, 2048, 1024, 512 or 256
// tokens, at most 256 blocks -- 64 at block size 1) that still gives at
// least kTargetWorkgroups decode workgroups on the vector-ALU decode (4 per
// CU on the chip's 256 CUs) or kTargetWorkgroupsMfma on the matrix-core
// decode (2 per CU; its workgroups are shorter-lived per token and all of
// them stay resident), so long sequences run few, long workgroups, a batch
// that fills the chip is not split (no merge launch), and short batches are
// cut until they fill it.
constexpr int kTargetWorkgroups = 1024;
constexpr int kTargetWorkgroupsMfma = 512;
constexpr int kPartitionChoices[] = {4096, 2048, 1024, 512, 256};

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Compiled instances.  Decode also takes block sizes below one wave-wide
// load (1 token per block); prefill needs a thread's 2 or 4 tile keys in
// one block.
bool supported_decode(int32_t head_dim, int32_t block_size) {
  return (head_dim == 64 || head_dim == 128) &&
         (block_size == 1 || block_size == 8 || block_size == 16 || block_size == 32);
}
bool supported_prefill(int32_t head_dim, int32_t block_size) {
  return (head_dim == 64 || head_dim == 128) &&
         (block_size == 8 || block_size == 16 || block_size == 32);
}

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Tokens per partition; 0 when the arguments are invalid.  A partition
// holds at most max_partition_blocks() blocks (four VGPRs of block ids per
// wave; one at block size 1).
int32_t partition_tokens(int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t block_size,
                         int32_t max_seq_len, int32_t requested) {
  if (block_size <= 0 || max_seq_len <= 0) return 0;
  const int group = (num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0)
                        ? num_q_heads / num_kv_heads
                        : 1;
  const int64_t cap = (int64_t)max_partition_blocks(block_size) * block_size;
  if (requested > 0)
    return (requested % block_size || requested > cap) ? 0 : requested;
  if (requested < 0) return 0;
  int64_t rows = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_q_heads > 0 ? num_q_heads : 1);
  if (num_q_heads > 0 && num_kv_heads > 0 && num_q_heads % num_kv_heads == 0)
    rows /= heads_per_workgroup(num_q_heads / num_kv_heads, block_size);
  const int64_t target =
      decode_on_mfma(group, block_size) ? kTargetWorkgroupsMfma : kTargetWorkgroups;
  int64_t part = 0;
  for (int choice : kPartitionChoices) {
    part = std::min<int64_t>(round_up(choice, block_size), cap);
    if (rows * ((max_seq_len + part - 1) / part) >= target) break;
  }
  if (max_seq_len <= part) part = round_up(max_seq_len, block_size);
  return (int32_t)part;
}

// Split-decode workspace: partial outputs, maxima and sums per (row,
// partition).  No state survives a call.
struct WorkspaceLayout {
  int32_t num_parts = 0;
  size_t o_off = 0, m_off = 0, l_off = 0, bytes = 0;
};

WorkspaceLayout layout(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                       int32_t max_seq_len, int32_t part) {
  WorkspaceLayout w;
  w.num_parts = (int32_t)((max_seq_len + (int64_t)part - 1) / part);
  if (w.num_parts <= 1) return w;
  const size_t heads = (size_t)num_seqs * num_q_heads;
  const size_t rows = heads * w.num_parts;
  w.o_off = 0;
  w.m_off = round_up((int64_t)(rows * head_dim * sizeof(float)), 256);
  w.l_off = w.m_off + round_up((int64_t)(rows * sizeof(float)), 256);
  w.bytes = w.l_off + round_up((int64_t)(rows * sizeof(float)), 256);
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

// Prefill key-range split.  Query tiles are 128 rows, key tiles 64 tokens.
// When the query tiles (x heads x chunks) are fewer than the workgroups the
// chip holds at once -- 256 CUs x 2 workgroups of the head-dim-128 kernel --
// part of the chip idles while each workgroup walks its whole key range.
// The key range of a query tile is then cut into parts of at least
// kMinSplitTiles tiles until the grid reaches about that many workgroups.
// Larger grids are not split, and a part holds at least kMinSplitTiles key
// tiles: the parts' partial outputs cost a write and a read of fp32 rows
// and a second launch, which shorter chains do not win back.
constexpr int kPrefillTargetWorkgroups = 512;
constexpr int kMinSplitTiles = 8;

struct PrefillSplit {
  int32_t parts = 1, tiles = 1;
  size_t o_off = 0, m_off = 0, l_off = 0, bytes = 0;
};

PrefillSplit prefill_split(int32_t num_chunks, int32_t total_q, int32_t max_q_len,
                           int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len) {
  PrefillSplit s;
  if (num_chunks <= 0 || total_q <= 0 || max_q_len <= 0 || num_q_heads <= 0 ||
      max_seq_len <= 0)
    return s;
  const int64_t base = ((int64_t)max_q_len + 127) / 128 * num_chunks * num_q_heads;
  const int64_t nt_max = ((int64_t)max_seq_len + 63) / 64;
  int64_t parts = (kPrefillTargetWorkgroups + base - 1) / base;
  parts = std::max<int64_t>(1, std::min<int64_t>(parts, nt_max / kMinSplitTiles));
  s.tiles = (int32_t)((nt_max + parts - 1) / parts);
  s.parts = (int32_t)((nt_max + s.tiles - 1) / s.tiles);
  if (s.parts <= 1) {
    s.parts = 1;
    s.tiles = (int32_t)std::max<int64_t>(nt_max, 1);
    return s;
  }
  const size_t rows = (size_t)s.parts * total_q * num_q_heads;
  s.o_off = 0;
  s.m_off = round_up((int64_t)(rows * head_dim * sizeof(float)), 256);
  s.l_off = s.m_off + round_up((int64_t)(rows * sizeof(float)), 256);
  s.bytes = s.l_off + round_up((int64_t)(rows * sizeof(float)), 256);
  return s;
}

}  // namespace

namespace {

// A pool argument as the kernel must address it: device memory as is,
// pinned host memory through its device mapping; anything else (pageable
// host memory) cannot be reached by a kernel.
bool kernel_address(const void *p, const void **out) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // an unknown pointer is not a launch failure
    return false;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
    *out = p;
    return true;
  }
  if (a.type == hipMemoryTypeHost && a.devicePointer) {
    *out = (const char *)a.devicePointer +
           ((const char *)p - (const char *)(a.hostPointer ? a.hostPointer : p));
    return true;
  }
  return false;
}

// Device scratch of pkv_paged_attention_decode_noalloc: the split
// partials of one call live in this file-scope array.  Each GPU the library
// runs on holds its own copy from the first such call until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is passed on.
static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (taken on its first use).
int device_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return PKV_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

bool copy_shape_ok(int32_t count, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t src_num_blocks, int32_t dst_num_blocks) {
  return count >= 0 && num_kv_heads > 0 && head_dim > 0 && head_dim % 8 == 0 &&
         block_size > 0 && src_num_blocks > 0 && dst_num_blocks > 0;
}

}  // namespace

extern "C" {

int pkv_kv_append(const void *key, const void *value, void *k_cache,
                  void *v_cache, const int32_t *slot_mapping,
                  int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks, void *stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || head_dim % 8)
    return PKV_ERR_INVALID;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return PKV_ERR_INVALID;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PKV_ERR_INVALID;
  AppendParams p;
  p.key = (const uint4 *)key;
  p.value = (const uint4 *)value;
  p.k_cache = (uint4 *)k_cache;
  p.v_cache = (uint4 *)v_cache;
  p.slots = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_kv_heads = num_kv_heads;
  p.chunks_per_row = head_dim / 8;
  p.block_size = block_size;
  p.num_slots = (int64_t)num_blocks * block_size;
  return hip_status(launch_kv_append(p, (hipStream_t)stream));
}

int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_seq_len,
                                  int32_t partition_size) {
  (void)head_dim;
  return partition_tokens(num_seqs, num_q_heads, num_kv_heads, block_size,
                          max_seq_len, partition_size);
}

size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_seq_len,
                                 int32_t partition_size) {
  const int32_t part = pkv_decode_partition_size(
      num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len,
      partition_size);
  if (part <= 0 || num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return layout(num_seqs, num_q_heads, head_dim, max_seq_len, part).bytes;
}

int pkv_paged_attention_decode(float *out, const void *q, const void *k_cache,
                               const void *v_cache,
                               const int32_t *block_tables,
                               const int32_t *seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_seq_len, float scale,
                               int32_t partition_size, const int32_t *seq_order,
                               void *workspace, size_t workspace_bytes,
                               void *stream) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_seq_len <= 0 || num_q_heads % num_kv_heads || !isfinite(scale) || !(scale > 0.f))
    return PKV_ERR_INVALID;
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_INVALID;
  if (!supported_decode(head_dim, block_size)) return PKV_ERR_UNSUPPORTED;
  const int32_t part = partition_tokens(num_seqs, num_q_heads, num_kv_heads,
                                        block_size, max_seq_len, partition_size);
  if (part <= 0) return PKV_ERR_INVALID;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
    return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PKV_ERR_INVALID;
  const WorkspaceLayout w =
      layout(num_seqs, num_q_heads, head_dim, max_seq_len, part);
  if (w.bytes > 0 && (!workspace || workspace_bytes < w.bytes ||
                      !aligned16(workspace)))
    return PKV_ERR_INVALID;

  DecodeParams p;
  p.out = out;
  p.q = (const _Float16 *)q;
  p.k_cache = (const _Float16 *)k_cache;
  p.v_cache = (const _Float16 *)v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  char *ws = (char *)workspace;
  p.ws_o = w.bytes ? (float *)(ws + w.o_off) : nullptr;
  p.ws_m = w.bytes ? (float *)(ws + w.m_off) : nullptr;
  p.ws_l = w.bytes ? (float *)(ws + w.l_off) : nullptr;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.part_tokens = part;
  p.num_parts = w.num_parts;
  p.scale_log2e = scale * kLog2e;
  // the dispatch order: a permutation of the batch, carried in the kernel
  // arguments (ignored for batches above kMaxOrderSeqs)
  p.has_order = 0;
  if (seq_order && num_seqs <= kMaxOrderSeqs) {
    bool seen[kMaxOrderSeqs] = {};
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t v = seq_order[i];
      if (v < 0 || v >= num_seqs || seen[v]) return PKV_ERR_INVALID;
      seen[v] = true;
      p.order[i] = (int16_t)v;
    }
    p.has_order = 1;
  }
  return hip_status(launch_decode(p, head_dim, block_size, (hipStream_t)stream));
}

int pkv_paged_attention_decode_noalloc(float *out, const void *q, const void *k_cache,
                                       const void *v_cache,
                                       const int32_t *block_tables,
                                       const int32_t *seq_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t max_seq_len, float scale,
                                       int32_t partition_size, const int32_t *seq_order,
                                       void *stream) {
  // The same argument checks and kernels as pkv_paged_attention_decode; the
  // partials go to the device's scratch array instead of a caller workspace.
  const size_t need = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                head_dim, block_size, max_seq_len,
                                                partition_size);
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    const int rc = device_scratch(&ws);
    if (rc != PKV_OK) return rc;
  }
  return pkv_paged_attention_decode(out, q, k_cache, v_cache, block_tables, seq_lens,
                                    num_seqs, num_q_heads, num_kv_heads, head_dim,
                                    block_size, num_blocks, max_blocks_per_seq, max_seq_len,
                                    scale, partition_size, seq_order, ws, need, stream);
}

size_t pkv_prefill_workspace_size(int32_t num_chunks, int32_t total_q_tokens,
                                  int32_t max_q_len, int32_t num_q_heads,
                                  int32_t head_dim, int32_t max_seq_len) {
  return prefill_split(num_chunks, total_q_tokens, max_q_len, num_q_heads, head_dim,
                       max_seq_len).bytes;
}

int pkv_paged_attention_prefill(float *out, const void *q,
                                const int32_t *cu_q_lens, const void *k_cache,
                                const void *v_cache,
                                const int32_t *block_tables,
                                const int32_t *seq_lens, int32_t num_chunks,
                                int32_t total_q_tokens, int32_t max_q_len,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, float scale, void *workspace,
                                size_t workspace_bytes, void *stream) {
  if (num_chunks < 0 || total_q_tokens < 0 || max_q_len < 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_seq_len <= 0 || num_q_heads % num_kv_heads || !isfinite(scale) ||
      !(scale > 0.f))
    return PKV_ERR_INVALID;
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size)
    return PKV_ERR_INVALID;
  if (num_q_heads > 65535 || num_chunks > 65535) return PKV_ERR_INVALID;
  if (!supported_prefill(head_dim, block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_chunks == 0 || total_q_tokens == 0) return PKV_OK;
  if (!out || !q || !cu_q_lens || !k_cache || !v_cache || !block_tables ||
      !seq_lens)
    return PKV_ERR_INVALID;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PKV_ERR_INVALID;
  PrefillParams p;
  p.out = out;
  p.q = (const _Float16 *)q;
  p.cu_q_lens = cu_q_lens;
  p.k_cache = (const _Float16 *)k_cache;
  p.v_cache = (const _Float16 *)v_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.num_chunks = num_chunks;
  p.total_q = total_q_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.scale_log2e = scale * kLog2e;
  const PrefillSplit sp = prefill_split(num_chunks, total_q_tokens, max_q_len, num_q_heads,
                                        head_dim, max_seq_len);
  p.num_splits = sp.parts;
  p.split_tiles = sp.tiles;
  p.ws_o = p.ws_m = p.ws_l = nullptr;
  if (sp.parts > 1) {
    if (!workspace || workspace_bytes < sp.bytes || !aligned16(workspace))
      return PKV_ERR_INVALID;
    char *w = (char *)workspace;
    p.ws_o = (float *)(w + sp.o_off);
    p.ws_m = (float *)(w + sp.m_off);
    p.ws_l = (float *)(w + sp.l_off);
  }
  return hip_status(launch_prefill(p, head_dim, block_size, max_q_len,
                                   (hipStream_t)stream));
}


int pkv_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                    const int32_t *src_blocks, const int32_t *dst_blocks,
                    int32_t count, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t src_num_blocks,
                    int32_t dst_num_blocks, void *stream) {
  if (!copy_shape_ok(count, num_kv_heads, head_dim, block_size, src_num_blocks,
                     dst_num_blocks))
    return PKV_ERR_INVALID;
  if (count == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !src_blocks || !dst_blocks)
    return PKV_ERR_INVALID;
  if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
    return PKV_ERR_INVALID;
  const void *a[6];
  const void *in[6] = {src_k, src_v, dst_k, dst_v, src_blocks, dst_blocks};
  for (int i = 0; i < 6; ++i)
    if (!kernel_address(in[i], &a[i])) return PKV_ERR_INVALID;
  CopyParams p;
  p.src_k = (const uint4 *)a[0];
  p.src_v = (const uint4 *)a[1];
  p.dst_k = (uint4 *)a[2];
  p.dst_v = (uint4 *)a[3];
  p.src_ids = (const int32_t *)a[4];
  p.dst_ids = (const int32_t *)a[5];
  p.count = count;
  p.src_num_blocks = src_num_blocks;
  p.dst_num_blocks = dst_num_blocks;
  p.chunks_per_block = (int64_t)num_kv_heads * block_size * head_dim / 8;
  return hip_status(launch_copy_blocks(p, (hipStream_t)stream));
}

int pkv_copy_blocks_dma(const void *src_k, const void *src_v, void *dst_k,
                        void *dst_v, const int32_t *src_blocks,
                        const int32_t *dst_blocks, int32_t count,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t src_num_blocks, int32_t dst_num_blocks,
                        void *stream) {
  if (!copy_shape_ok(count, num_kv_heads, head_dim, block_size, src_num_blocks,
                     dst_num_blocks))
    return PKV_ERR_INVALID;
  if (count == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !src_blocks || !dst_blocks)
    return PKV_ERR_INVALID;
  for (int32_t i = 0; i < count; ++i)
    if (src_blocks[i] < 0 || src_blocks[i] >= src_num_blocks || dst_blocks[i] < 0 ||
        dst_blocks[i] >= dst_num_blocks)
      return PKV_ERR_INVALID;
  const size_t bytes = (size_t)num_kv_heads * block_size * head_dim * 2;
  hipStream_t st = (hipStream_t)stream;
  for (int32_t i = 0; i < count;) {
    // one copy per run of blocks consecutive on both sides
    int32_t n = 1;
    while (i + n < count && src_blocks[i + n] == src_blocks[i] + n &&
           dst_blocks[i + n] == dst_blocks[i] + n)
      ++n;
    const size_t so = (size_t)src_blocks[i] * bytes, dof = (size_t)dst_blocks[i] * bytes;
    hipError_t e = hipMemcpyAsync((char *)dst_k + dof, (const char *)src_k + so,
                                  n * bytes, hipMemcpyDefault, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync((char *)dst_v + dof, (const char *)src_v + so, n * bytes,
                         hipMemcpyDefault, st);
    if (e != hipSuccess) return PKV_ERR_HIP;
    i += n;
  }
  return PKV_OK;
}

}  // extern "C"
