// Device helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Makes a value the compiler treats as divergent wave-uniform (e.g. the
// wave index), so that loads addressed by it become scalar loads.
__device__ __forceinline__ int uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// DPP move of a float within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}

// Sum over aligned groups of LANES (8 or 16) consecutive lanes; every lane
// of a group receives the group's sum.  quad_perm swaps pairs, then pairs of
// pairs; half-row mirror folds quads into 8-lane halves; row mirror folds
// the two halves of a 16-lane row.
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(LANES == 8 || LANES == 16, "group of 8 or 16 lanes");
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  if constexpr (LANES == 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, kWave);
}

// IEEE maximum (NaN-propagating): lowers to v_maximum3_f32 on gfx950 with no
// operand canonicalisation, unlike fmaxf (maxNum) on values of unknown origin
// such as MFMA results.
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Reductions over the four lanes l, l^16, l^32, l^48 with the gfx950 row
// swaps (VALU, no LDS round trip): v_permlane32_swap exchanges the upper
// half of one copy with the lower half of the other, so the two results hold
// both halves' values at every lane; v_permlane16_swap does the same for odd
// and even 16-lane rows.
__device__ __forceinline__ float max_over_rows(float v) {
  const unsigned u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float v) {
  const unsigned u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

__device__ __forceinline__ uint4 ld16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// 16-byte load with the nontemporal hint: data streamed once (the K/V rows
// of a decode) should not displace reusable lines in the caches.
typedef unsigned u4v_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void *p) {
  const u4v_t v = __builtin_nontemporal_load(reinterpret_cast<const u4v_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
typedef unsigned u2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8_nt(const void *p) {
  const u2v_t v = __builtin_nontemporal_load(reinterpret_cast<const u2v_t *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void st16(void *p, uint4 v) {
  *reinterpret_cast<uint4 *>(p) = v;
}

__device__ __forceinline__ h8_t as_h8(uint4 v) {
  return __builtin_bit_cast(h8_t, v);
}

// q . k over 8 fp16 pairs, fp32 accumulation (v_dot2c_f32_f16).
__device__ __forceinline__ float dot8(h8_t a, h8_t b, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1),
                               __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3),
                               __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5),
                               __builtin_shufflevector(b, b, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7),
                               __builtin_shufflevector(b, b, 6, 7), acc, false);
  return acc;
}

// Block ids of one decode partition of up to 64 * N blocks, N per lane:
// lane l keeps entries l, 64 + l, ..., read back wave-uniformly with
// v_readlane.  issue() loads them (clamped, always in bounds) before the
// partition's length is known; settle() then replaces entries outside the
// pool with 0 and reports whether a live entry (index < nb) was one.
template <int N>
struct PartitionIds {
  int v[N];
  __device__ __forceinline__ void issue(const int32_t *trow, int blk0, int max_blocks,
                                        int lane) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = trow[min(blk0 + kWave * i + lane, max_blocks - 1)];
  }
  __device__ __forceinline__ bool settle(int nb, int num_blocks, int lane) {
    bool bad = false;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool out = v[i] < 0 || v[i] >= num_blocks;
      bad |= kWave * i + lane < nb && out;
      if (out || kWave * i + lane >= nb) v[i] = 0;
    }
    return bad;
  }
  // entry j of the partition, j wave-uniform and < 64 * N
  __device__ __forceinline__ int get(int j) const {
    int r = __builtin_amdgcn_readlane(v[0], j & (kWave - 1));
#pragma unroll
    for (int i = 1; i < N; ++i)
      if (j >= kWave * i) r = __builtin_amdgcn_readlane(v[i], j & (kWave - 1));
    return r;
  }
};

// v_mfma_f32_16x16x32_f16: D(16x16) = A(16x32) B(32x16) + C.  Lane l
// supplies row l%16 of A and column l%16 of B, each as 8 fp16 values of the
// contraction index (group l/16); lane l receives D rows 4*(l/16)+r, r<4,
// of column l%16.
__device__ __forceinline__ f4_t mfma16x16x32(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace pkv
