// Streaming-read reference kernel for measurements (not part of the
// paged-attention library): reads a contiguous buffer once with 16-byte
// nontemporal loads, the same load form the decode uses on its K/V rows, so
// that a decode's bandwidth can be set against what a plain sequential read
// of HBM reaches on the same device.  Built into its own library.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned int u4v_t __attribute__((ext_vector_type(4)));

// Two streams, the two halves of the buffer, read grid-stride over 16-byte
// chunks with four loads from each in flight per thread and iteration (a
// chunk count that is odd leaves one last chunk, read by thread 0).  The
// loaded words are folded into one value that is written only when it
// equals an arbitrary constant, which keeps the loads alive without a store
// per thread.
__global__ __launch_bounds__(256) void stream_read_kernel(const u4v_t *__restrict__ p,
                                                          uint64_t n, uint32_t *sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t h = n / 2;
  const u4v_t *__restrict__ q = p + h;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u4v_t acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < h; i += 4 * stride) {
    const u4v_t a0 = __builtin_nontemporal_load(p + i);
    const u4v_t b0 = __builtin_nontemporal_load(q + i);
    const u4v_t a1 = __builtin_nontemporal_load(p + i + stride);
    const u4v_t b1 = __builtin_nontemporal_load(q + i + stride);
    const u4v_t a2 = __builtin_nontemporal_load(p + i + 2 * stride);
    const u4v_t b2 = __builtin_nontemporal_load(q + i + 2 * stride);
    const u4v_t a3 = __builtin_nontemporal_load(p + i + 3 * stride);
    const u4v_t b3 = __builtin_nontemporal_load(q + i + 3 * stride);
    acc ^= (a0 ^ b0) ^ (a1 ^ b1) ^ (a2 ^ b2) ^ (a3 ^ b3);
  }
  for (; i < h; i += stride)
    acc ^= __builtin_nontemporal_load(p + i) ^ __builtin_nontemporal_load(q + i);
  if ((n & 1) && blockIdx.x == 0 && threadIdx.x == 0) acc ^= p[n - 1];
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x9e3779b9u) sink[0] = v;
}

}  // namespace

// Enqueues one read of `bytes` bytes at `buf` (device memory, 16-byte
// aligned, bytes a multiple of 16) on `stream` with `blocks` workgroups of
// 256 threads.  `sink` is one device uint32 the kernel may write.  Returns
// a hipError_t value (0 on success); invalid arguments give
// hipErrorInvalidValue and enqueue nothing.
extern "C" int pkvb_stream_read(const void *buf, uint64_t bytes, uint32_t *sink,
                                int32_t blocks, void *stream) {
  if (!buf || !sink || blocks <= 0 || bytes == 0 || (bytes & 15u) ||
      ((uintptr_t)buf & 15u))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0,
                     (hipStream_t)stream, (const u4v_t *)buf, bytes / 16, sink);
  return (int)hipGetLastError();
}
