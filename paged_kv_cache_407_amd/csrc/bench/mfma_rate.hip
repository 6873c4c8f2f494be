// Matrix-core reference kernel for measurements (not part of the
// paged-attention library): every wave issues independent chains of one fp16
// MFMA shape back to back, with nothing else in its loop, so that the prefill's
// FLOP rate can be set against what that instruction sustains on the same
// device and clock.  Built into the measurement library with the streaming
// read.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef float f16_t __attribute__((ext_vector_type(16)));

// A operands are all `va`, B operands all `vb` (fp16), in separate registers
// as in the prefill (an MFMA that reads A and B from the same registers runs
// slower); with va = vb = 1/8 every product and partial sum is exact, so each
// output element is a closed form of iters, the chain count and the
// contraction length (the GPU test checks it).
template <int NACC>
__global__ __launch_bounds__(256) void mfma16x16x32_kernel(float *out, int iters, float va,
                                                              float vb) {
  h8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)va;
    b[i] = (_Float16)vb;
  }
  f4_t acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = f4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <int NACC>
__global__ __launch_bounds__(256) void mfma32x32x16_kernel(float *out, int iters, float va,
                                                              float vb) {
  h8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)va;
    b[i] = (_Float16)vb;
  }
  f16_t acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Independent accumulator chains per wave of each shape (enough to cover the
// MFMA result latency).  The library is built with the accumulators in
// ordinary VGPRs, as the prefill keeps them: in accumulation registers the
// compiler rotates the 16x16x32 chains through different register tuples
// each iteration and adds dozens of register moves to the loop.
constexpr int kChains16 = 8, kChains32 = 4;

// Enqueues `blocks` workgroups of 256 threads on `stream`; each wave runs
// `iters` iterations of its chains of one MFMA shape, all A operands `va`
// and all B operands `vb` (rounded to fp16): shape 0 is
// v_mfma_f32_16x16x32_f16 (kChains16 chains), shape 1 v_mfma_f32_32x32x16_f16
// (kChains32 chains).  `out` (device, blocks * 256 floats) receives one sum of
// accumulators per thread.  Returns a hipError_t value (0 on success);
// invalid arguments give hipErrorInvalidValue and enqueue nothing.
extern "C" int pkvb_mfma_rate(float *out, int32_t shape, int32_t blocks, int32_t iters,
                              float va, float vb, void *stream) {
  if (!out || blocks <= 0 || iters <= 0 || (shape != 0 && shape != 1))
    return (int)hipErrorInvalidValue;
  if (shape == 0)
    hipLaunchKernelGGL(mfma16x16x32_kernel<kChains16>, dim3(blocks), dim3(256), 0,
                       (hipStream_t)stream, out, iters, va, vb);
  else
    hipLaunchKernelGGL(mfma32x32x16_kernel<kChains32>, dim3(blocks), dim3(256), 0,
                       (hipStream_t)stream, out, iters, va, vb);
  return (int)hipGetLastError();
}
