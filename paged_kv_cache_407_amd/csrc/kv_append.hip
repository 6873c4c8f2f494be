// kv append: each new token's K and V rows are copied, bit for bit, into the
// physical slot its slot id names -- block slot / block_size, offset
// slot % block_size ("LLM 推理引擎 Continuous Batching 与 PagedAttention：
// 从 vLLM 原理到生产级部署实战", §3.2 BlockManager.append_token).
//
// One thread moves one 16-byte chunk (8 fp16) of one (token, head) row, so a
// wave moves 1 KB of contiguous source per instruction and each row lands as
// D*2 contiguous bytes of its block.  Pure HBM copy: 2 * 2 * T * Hkv * D bytes
// read and written.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total =
      (int64_t)p.num_tokens * p.num_kv_heads * p.chunks_per_row;
  if (i >= total) return;
  const int c = (int)(i % p.chunks_per_row);
  const int64_t r = i / p.chunks_per_row;
  const int h = (int)(r % p.num_kv_heads);
  const int t = (int)(r / p.num_kv_heads);
  const int32_t slot = p.slots[t];
  if (slot < 0 || slot >= p.num_slots) return;  // padding row / out of pool
  const int64_t blk = slot / p.block_size;
  const int64_t off = slot % p.block_size;
  const int64_t dst =
      ((blk * p.num_kv_heads + h) * p.block_size + off) * p.chunks_per_row + c;
  const uint4 kv = p.key[i];
  const uint4 vv = p.value[i];
  p.k_cache[dst] = kv;
  p.v_cache[dst] = vv;
}

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream) {
  const int64_t total =
      (int64_t)p.num_tokens * p.num_kv_heads * p.chunks_per_row;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  kv_append_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace pkv
