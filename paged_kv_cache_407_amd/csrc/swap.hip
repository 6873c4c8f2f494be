// Whole-block copies between two KV pools: the data movement of swapping a
// request's KV cache out to host memory and back ("LLM 推理引擎 Continuous
// Batching 与 PagedAttention：从 vLLM 原理到生产级部署实战", §4.4 Swap: a
// request's GPU blocks are copied to CPU blocks and freed, later copied back
// into newly taken GPU blocks).  The same copy serves any pair of pools:
// device -> pinned host (swap out), pinned host -> device (swap in), device
// -> device (duplicating blocks).
//
// A block of one pool is [num_kv_heads][block_size][head_dim] fp16 for K and
// the same for V, contiguous in both pools (their layout is the cache
// layout), so a block pair is two contiguous copies of block_bytes.  One
// workgroup moves a 16 KB slice of one block pair's K and V: every thread
// issues its four 16-byte loads per tensor before any store, so a wave keeps
// 8 KB in flight.  Over PCIe the rate is bound by the link; between device
// pools it is an HBM copy.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int kCopyChunksPerThread = 4;
constexpr int kCopySlice = kCopyThreads * kCopyChunksPerThread;  // 16-byte chunks

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyParams p) {
  const int64_t slices = (p.chunks_per_block + kCopySlice - 1) / kCopySlice;
  const int64_t pair = blockIdx.x / slices;
  const int64_t slice = blockIdx.x % slices;
  const int32_t s = p.src_ids[pair], d = p.dst_ids[pair];
  if (s < 0 || s >= p.src_num_blocks || d < 0 || d >= p.dst_num_blocks) return;
  const uint4 *sk = p.src_k + (int64_t)s * p.chunks_per_block;
  const uint4 *sv = p.src_v + (int64_t)s * p.chunks_per_block;
  uint4 *dk = p.dst_k + (int64_t)d * p.chunks_per_block;
  uint4 *dv = p.dst_v + (int64_t)d * p.chunks_per_block;
  const int64_t c0 = slice * kCopySlice + threadIdx.x;
  uint4 k[kCopyChunksPerThread], v[kCopyChunksPerThread];
#pragma unroll
  for (int j = 0; j < kCopyChunksPerThread; ++j) {
    const int64_t c = c0 + (int64_t)j * kCopyThreads;
    if (c < p.chunks_per_block) {
      k[j] = sk[c];
      v[j] = sv[c];
    }
  }
#pragma unroll
  for (int j = 0; j < kCopyChunksPerThread; ++j) {
    const int64_t c = c0 + (int64_t)j * kCopyThreads;
    if (c < p.chunks_per_block) {
      dk[c] = k[j];
      dv[c] = v[j];
    }
  }
}

hipError_t launch_copy_blocks(const CopyParams &p, hipStream_t stream) {
  if (p.count == 0) return hipSuccess;
  const int64_t slices = (p.chunks_per_block + kCopySlice - 1) / kCopySlice;
  const int64_t grid = slices * p.count;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  copy_blocks_kernel<<<dim3((unsigned)grid), dim3(kCopyThreads), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pkv
