// Paged attention decode on the vector ALUs.
//
// What is computed ("LLM 推理引擎 Continuous Batching 与 PagedAttention：从
// vLLM 原理到生产级部署实战", §3.3): for each sequence and query head, the
// scores q.k_t * scale over the sequence's tokens, reached through the block
// table (logical block t / block_size -> physical block, at most
// min(block_size, seq_len - block start) tokens in a block), the running
// maximum and sum of exponentials, and the value rows weighted by the
// normalised exponentials (the page leaves that last step out; this is its
// plain reading).
//
// Design for CDNA4 (wave64): a token row of D fp16 is D/8 lanes x 16 bytes,
// so one wave-wide 16-byte load reads 64/(D/8) whole rows -- 1 KB of a
// block's contiguous [block_size][D] tile per instruction, fully coalesced.
// Each lane keeps 8 query values, takes 8-wide dot products with
// v_dot2c_f32_f16 and the row sum is finished with DPP inside each row
// group.  Every lane therefore owns the scores of the very tokens whose V
// slices it holds, so the PV step needs no data exchange.  Softmax runs in
// base 2 with scale*log2(e) folded into the scores.  Tokens past seq_len are
// removed by selecting (never by multiplying: the tail slots may hold NaN).
//
// A sequence is cut into partitions of part_tokens; one workgroup of 4 waves
// takes one (partition, sequence, query head).  Waves take interleaved steps
// of CH blocks (8 KB of K and 8 KB of V in flight per wave and step), keep a
// running max / sum / accumulator, and are merged through LDS.  With several
// partitions the workgroup writes (max, sum, unnormalised output) and
// decode_merge_kernel combines them: M = max_i m_i, out = sum_i 2^(m_i-M) o_i
// / sum_i 2^(m_i-M) l_i -- the same rescaling the running recurrence uses,
// applied across partitions.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

template <int D, int BS>
struct DecodeShape {
  static constexpr int LPR = D / 8;        // lanes per token row
  static constexpr int RPL = kWave / LPR;  // token rows per wave-wide load
  static constexpr int LPB = BS / RPL;     // loads per lane per block
  static constexpr int CH = LPB >= 8 ? 1 : 8 / LPB;  // blocks per wave step
  static constexpr int NL = CH * LPB;      // 16-byte loads per lane per step
  static_assert(BS % RPL == 0, "block must hold whole wave loads");
};

template <int D, int BS>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeParams p) {
  using Sh = DecodeShape<D, BS>;
  constexpr int LPR = Sh::LPR, RPL = Sh::RPL, LPB = Sh::LPB, CH = Sh::CH,
                NL = Sh::NL;
  __shared__ float s_acc[4][D];
  __shared__ float s_m[4], s_l[4];
  __shared__ int s_bad[4];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  int idx = blockIdx.x;
  const int h = idx % p.num_q_heads;
  idx /= p.num_q_heads;
  const int s = idx % p.num_seqs;
  const int part = idx / p.num_seqs;

  const int L = p.seq_lens[s];
  const size_t row = (size_t)s * p.num_q_heads + h;
  const bool len_ok =
      L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS;
  if (!len_ok) {
    // With a split, the merge kernel writes this row.
    if (p.num_parts == 1 && part == 0)
      for (int d = threadIdx.x; d < D; d += blockDim.x)
        p.out[row * D + d] = __builtin_nanf("");
    return;
  }
  if (part >= cdiv(L, p.part_tokens)) return;

  const int kvh = h / p.group;
  const int part_blocks = p.part_tokens / BS;
  const int nblk = cdiv(L, BS);
  const int blk0 = part * part_blocks;
  const int blk1 = min(blk0 + part_blocks, nblk);
  // Tokens of this partition; a wave step may overhang the partition's last
  // block, and those zero-filled rows must not enter the softmax.
  const int tok_end = min(L, blk1 * BS);
  const int32_t *trow = p.block_tables + (size_t)s * p.max_blocks_per_seq;

  const int col = lane % LPR;   // 16-byte column within a token row
  const int rrow = lane / LPR;  // token row within one wave-wide load
  const h8_t qv = as_h8(ld16(p.q + row * D + col * 8));

  float m = -INFINITY, lsum = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  int bad = 0;
  const size_t head_elems = (size_t)BS * D;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  for (int b = blk0 + wave * CH; b < blk1; b += 4 * CH) {
    uint4 kr[NL], vr[NL];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int bb = b + c;
      int phys = 0;
      if (bb < blk1) {
        phys = trow[bb];
        if (phys < 0 || phys >= p.num_blocks) {
          bad = 1;
          phys = 0;
        }
      }
      const size_t base =
          ((size_t)phys * p.num_kv_heads + kvh) * head_elems + rrow * D + col * 8;
#pragma unroll
      for (int j = 0; j < LPB; ++j) {
        if (bb < blk1) {
          kr[c * LPB + j] = ld16(p.k_cache + base + (size_t)j * RPL * D);
          vr[c * LPB + j] = ld16(p.v_cache + base + (size_t)j * RPL * D);
        } else {
          kr[c * LPB + j] = zero;
          vr[c * LPB + j] = zero;
        }
      }
    }
    float sc[NL];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int tok = (b + i / LPB) * BS + (i % LPB) * RPL + rrow;
      const float d = group_sum<LPR>(dot8(qv, as_h8(kr[i]), 0.f));
      sc[i] = tok < tok_end ? d * p.scale_log2e : -INFINITY;
      cmax = fmaxf(cmax, sc[i]);
    }
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) cmax = xor_max(cmax, off);
    const float mnew = fmaxf(m, cmax);
    const float alpha = fast_exp2(m - mnew);
    lsum *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= alpha;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int tok = (b + i / LPB) * BS + (i % LPB) * RPL + rrow;
      const bool ok = tok < tok_end;
      const float pr = ok ? fast_exp2(sc[i] - mnew) : 0.f;
      const h8_t v = as_h8(ok ? vr[i] : zero);
      lsum += pr;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(pr, (float)v[k], acc[k]);
    }
    m = mnew;
  }

  // Lanes of one row group hold equal sums; add the row groups.
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    lsum = xor_sum(lsum, off);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = xor_sum(acc[k], off);
  }
  if (lane < LPR) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s_acc[wave][col * 8 + k] = acc[k];
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = lsum;
    s_bad[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = fast_exp2(s_m[w] - M);  // an idle wave has m = -inf
      o = fmaf(e, s_acc[w][d], o);
      l = fmaf(e, s_l[w], l);
    }
    if (s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3]) o = __builtin_nanf("");
    if (p.num_parts == 1) {
      p.out[row * D + d] = o / l;
    } else {
      const size_t pi = row * p.num_parts + part;
      p.ws_o[pi * D + d] = o;
      if (d == 0) {
        p.ws_m[pi] = M;
        p.ws_l[pi] = l;
      }
    }
  }
}

template <int D, int BS>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  const size_t row = blockIdx.x;
  const int s = (int)(row / p.num_q_heads);
  const int d = threadIdx.x;
  const int L = p.seq_lens[s];
  const bool len_ok =
      L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS;
  if (!len_ok) {
    p.out[row * D + d] = __builtin_nanf("");
    return;
  }
  const int np = cdiv(L, p.part_tokens);
  const size_t base = row * p.num_parts;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, p.ws_m[base + i]);
  float o = 0.f, l = 0.f;
  for (int i = 0; i < np; ++i) {
    const float e = fast_exp2(p.ws_m[base + i] - M);
    o = fmaf(e, p.ws_o[(base + i) * D + d], o);
    l = fmaf(e, p.ws_l[base + i], l);
  }
  p.out[row * D + d] = o / l;
}

template <int D, int BS>
static hipError_t launch(const DecodeParams &p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads;
  const int64_t grid = rows * p.num_parts;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  decode_partition_kernel<D, BS><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_parts == 1) return e;
  decode_merge_kernel<D, BS><<<dim3((unsigned)rows), dim3(D), 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams &p, int head_dim, int block_size,
                         hipStream_t stream) {
  if (head_dim == 128 && block_size == 16) return launch<128, 16>(p, stream);
  if (head_dim == 128 && block_size == 32) return launch<128, 32>(p, stream);
  if (head_dim == 64 && block_size == 16) return launch<64, 16>(p, stream);
  if (head_dim == 64 && block_size == 32) return launch<64, 32>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
