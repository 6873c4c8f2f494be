// Paged attention prefill of causal chunks on MFMA.
//
// What is computed ("LLM 推理引擎 Continuous Batching 与 PagedAttention：从
// vLLM 原理到生产级部署实战", §4.3 Chunked Prefill, with the causal rule of
// the prefill phase in §1.1): a chunk of C new tokens sits on a prefix of P
// tokens that is already in paged blocks; query row j of the chunk is token
// P + j of its sequence and attends to keys 0 .. P + j, read through the
// block table exactly as the decode does.
//
// Design for CDNA4: one workgroup of 4 waves takes a 64-row query tile of one
// (chunk, head); each wave owns 16 query rows.  Key/value tiles of 64 tokens
// are gathered block by block (one block-table lookup per block) from HBM
// into LDS with 16-byte loads.  Per tile and wave:
//   S^T = K Q^T    (v_mfma_f32_16x16x32_f16; A = 16 keys x 32 dims from LDS,
//                   B = the wave's 16 query rows, kept in registers)
//   online softmax (base 2, running max and sum per query row; the row's
//                   values sit in the 4 lanes l%16 = row, so the max and sum
//                   need two cross-lane steps)
//   O^T += V^T P^T (the accumulator layout of S^T is exactly the B-operand
//                   layout of P^T, so the fp16 weights never leave their
//                   lanes; V^T is read from the row-major V tile in LDS).
// Computing the transposed products keeps each query row's statistics and
// its output columns in the same lanes, so the rescale by 2^(m_old - m_new)
// needs no exchange.  Keys above the diagonal are removed by selection;
// tiles wholly above it are never loaded.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

template <int D, int BS>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int BM = 64, BN = 64;
  constexpr int KS = D / 32;        // MFMA steps over the head dimension
  constexpr int DT = D / 16;        // 16-wide output column tiles
  constexpr int CPR = D / 8;        // 16-byte chunks per token row
  constexpr int STR = D + 8;        // LDS row stride in fp16 (16-byte pad)
  constexpr int NCH = BN * CPR / 256;
  constexpr int NBT = BN / BS;      // blocks per key tile
  static_assert(NCH * 256 == BN * CPR, "tile load split");
  __shared__ __attribute__((aligned(16))) _Float16 sK[BN * STR];
  __shared__ __attribute__((aligned(16))) _Float16 sV[BN * STR];
  __shared__ int sPhys[NBT];
  __shared__ int sBad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int qt = blockIdx.x, h = blockIdx.y, c = blockIdx.z;
  const int q_begin = p.cu_q_lens[c], q_end = p.cu_q_lens[c + 1];
  if (q_begin < 0 || q_end > p.total_q || q_end < q_begin) return;
  const int qlen = q_end - q_begin;
  const int row0 = qt * BM;
  if (row0 >= qlen) return;
  const int L = p.seq_lens[c];
  const int P = L - qlen;
  const int Hq = p.num_q_heads;

  if (!(P >= 0 && L >= 1 && L <= p.max_blocks_per_seq * BS)) {
    for (int i = tid; i < BM * D; i += 256) {
      const int r = row0 + i / D;
      if (r < qlen)
        p.out[((size_t)(q_begin + r) * Hq + h) * D + i % D] = __builtin_nanf("");
    }
    return;
  }

  const int g = lane >> 4;          // contraction group of this lane
  const int lc = lane & 15;         // row / column index of this lane
  const int qr = row0 + wave * 16 + lc;   // query row (within the chunk)
  const int qpos = P + qr;                // its position in the sequence
  const int kvh = h / p.group;
  const int kv_end = P + min(row0 + BM, qlen);
  const int ntiles = cdiv(kv_end, BN);
  const int32_t *trow = p.block_tables + (size_t)c * p.max_blocks_per_seq;

  h8_t qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (qr < qlen)
      v = ld16(p.q + ((size_t)(q_begin + qr) * Hq + h) * D + 32 * kk + 8 * g);
    qf[kk] = as_h8(v);
  }

  f4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  if (tid == 0) sBad = 0;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int kbase = kt * BN;
    __syncthreads();  // the previous tile is consumed
    if (tid < NBT) {
      const int pos = kbase + tid * BS;
      int ph = -1;
      if (pos < L) {
        ph = trow[pos / BS];
        if (ph < 0 || ph >= p.num_blocks) {
          sBad = 1;
          ph = -1;
        }
      }
      sPhys[tid] = ph;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int id = tid + 256 * i;
      const int t = id / CPR, cc = id % CPR;
      const int pos = kbase + t;
      const int ph = sPhys[t / BS];
      uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
      if (pos < L && ph >= 0) {
        const size_t off =
            (((size_t)ph * p.num_kv_heads + kvh) * BS + pos % BS) * D + cc * 8;
        kv = ld16(p.k_cache + off);
        vv = ld16(p.v_cache + off);
      }
      st16(&sK[t * STR + cc * 8], kv);
      st16(&sV[t * STR + cc * 8], vv);
    }
    __syncthreads();

    // S^T for 4 sub-tiles of 16 keys: lane holds keys kbase+16mm+4g+r of
    // query row lc.
    f4_t st[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      st[mm] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const h8_t a = as_h8(ld16(&sK[(16 * mm + lc) * STR + 32 * kk + 8 * g]));
        st[mm] = mfma16x16x32(a, qf[kk], st[mm]);
      }
    }
    float sv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kpos = kbase + 16 * mm + 4 * g + r;
        const float x = st[mm][r] * p.scale_log2e;
        sv[mm * 4 + r] = kpos <= qpos ? x : -INFINITY;
        tmax = fmaxf(tmax, sv[mm * 4 + r]);
      }
    }
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
    const float mnew = fmaxf(m, tmax);   // key 0 is always visible: finite
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    h8_t pb[2];
    float psum = 0.f;
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kpos = kbase + 16 * mm + 4 * g + r;
        const float pr = kpos <= qpos ? fast_exp2(sv[mm * 4 + r] - mnew) : 0.f;
        const _Float16 ph = (_Float16)pr;
        psum += (float)ph;
        pb[mm >> 1][(mm & 1) * 4 + r] = ph;
      }
    }
    l = l * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    // O^T[d][row] += sum_k V[k][d] P[row][k]; contraction slot 8g+r is key
    // 32ks+4g+r, slot 8g+4+r is key 32ks+16+4g+r (matching pb's layout).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        h8_t a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a[r] = sV[(32 * ks + 4 * g + r) * STR + 16 * dt + lc];
          a[4 + r] = sV[(32 * ks + 16 + 4 * g + r) * STR + 16 * dt + lc];
        }
        o[dt] = mfma16x16x32(a, pb[ks], o[dt]);
      }
    }
  }

  l = xor_sum(l, 16);
  l = xor_sum(l, 32);
  if (qr < qlen) {
    float *orow = p.out + ((size_t)(q_begin + qr) * Hq + h) * D;
    const bool bad = sBad != 0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f4_t r = o[dt] / l;
      if (bad) r = f4_t{__builtin_nanf(""), __builtin_nanf(""),
                        __builtin_nanf(""), __builtin_nanf("")};
      *reinterpret_cast<f4_t *>(orow + 16 * dt + 4 * g) = r;
    }
  }
}

template <int D, int BS>
static hipError_t launch(const PrefillParams &p, int max_q_len,
                         hipStream_t stream) {
  if (p.num_chunks == 0 || max_q_len == 0) return hipSuccess;
  const dim3 grid(cdiv(max_q_len, 64), p.num_q_heads, p.num_chunks);
  prefill_kernel<D, BS><<<grid, dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams &p, int head_dim, int block_size,
                          int max_q_len, hipStream_t stream) {
  if (head_dim == 128 && block_size == 16) return launch<128, 16>(p, max_q_len, stream);
  if (head_dim == 128 && block_size == 32) return launch<128, 32>(p, max_q_len, stream);
  if (head_dim == 64 && block_size == 16) return launch<64, 16>(p, max_q_len, stream);
  if (head_dim == 64 && block_size == 32) return launch<64, 32>(p, max_q_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
