// Paged attention decode: on the vector ALUs for one or two query heads per
// KV head (and at block size 1), on the matrix cores when a workgroup serves
// 4, 8 or 16 query heads of one KV head at block size 8, 16 or 32.
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
// Design for CDNA4 (wave64):
// * A token row of D fp16 is D/8 lanes x 16 bytes, so one wave-wide 16-byte
//   load reads 64/(D/8) whole rows -- 1 KB of a block's contiguous
//   [block_size][D] tile per instruction.  K/V rows are used once, so they
//   are loaded with the nontemporal hint.
// * One workgroup serves GH query heads that share one KV head (grouped
//   query attention), so a K/V row is read from HBM once for all of them.
//   Each lane keeps 8 query values per head, takes 8-wide dot products with
//   v_dot2c_f32_f16 and finishes each row sum with DPP inside its row group;
//   every lane then owns the scores of exactly the tokens whose V slices it
//   holds, so the PV step needs no data exchange.
// * Softmax runs in base 2 with scale*log2(e) folded into the scores.  Tokens
//   past the partition's end are removed by selecting (never by multiplying:
//   tail slots may hold NaN).
// * A sequence is cut into partitions of part_tokens (at most 256 blocks, so
//   four VGPRs hold the partition's block ids: lane j keeps entries j,
//   64 + j, ... and a wave reads them with v_readlane; for blocks smaller
//   than one wave-wide load, at most 64 blocks, and each lane fetches its
//   token's entry with a lane permute).  One workgroup of 8 waves (fewer
//   when a partition holds fewer wave steps) takes one (partition,
//   sequence, head group); waves take interleaved steps of whole blocks and
//   are merged through LDS.
// * With several partitions, each workgroup stores (max, sum, unnormalised
//   output) and decode_merge_kernel combines them: M = max_i m_i,
//   out = sum_i 2^(m_i-M) o_i / sum_i 2^(m_i-M) l_i -- the rescaling of the
//   running recurrence, applied across partitions.  (Merging inside the last
//   partition to finish would need device-scope release/acquire fences,
//   which on this chip write back and invalidate the L2 of every XCD per
//   workgroup; a second launch is far cheaper.)
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

// log2 of the largest softmax weight tolerated before a running maximum is
// moved
constexpr float kLazyRescale = 8.f;

// Tuning constants: waves per workgroup (where a partition holds enough wave
// steps), and 16-byte K loads per lane in one wave step (the same number of V
// loads is in flight beside them).
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 8
#endif
#ifndef PKV_DECODE_STEP_LOADS
#define PKV_DECODE_STEP_LOADS 8
#endif
constexpr int kDecodeWaves = PKV_DECODE_WAVES;
constexpr int kStepLoads = PKV_DECODE_STEP_LOADS;

// Wave step layout.  Load i of a step that starts at block b brings token
// b*BS + i*RPL + r to the lanes of row r.  When a block holds whole
// wave-wide loads (BS >= RPL) every load reads one block, whose id is
// wave-uniform; smaller blocks (SUB) put RPL/BS blocks in one load and each
// lane fetches the id of its own token's block.
template <int D, int BS>
struct DecodeShape {
  static constexpr int LPR = D / 8;        // lanes per token row
  static constexpr int RPL = kWave / LPR;  // token rows per wave-wide load
  static constexpr bool SUB = BS < RPL;
  static constexpr int LPB = SUB ? 1 : BS / RPL;  // loads per lane per block
  static constexpr int NL = SUB ? kStepLoads
                                : (LPB >= kStepLoads ? LPB : (kStepLoads / LPB) * LPB);
  static constexpr int BPS = NL * RPL / BS;       // blocks per wave step
  static_assert(SUB ? RPL % BS == 0 : BS % RPL == 0, "blocks and loads nest");
  // Waves per workgroup: a partition holds at most kMaxPartBlocks blocks, so
  // with blocks smaller than a wave-wide load it holds only a few wave steps
  // (2 at head_dim 128, 1 at 64); more waves would idle.
  static constexpr int STEPS = kMaxPartBlocks / BPS;  // wave steps per partition
  static constexpr int NW = STEPS < kDecodeWaves ? (STEPS > 0 ? STEPS : 1) : kDecodeWaves;
};

template <int D, int BS, int GH>
__global__ __launch_bounds__((64 * DecodeShape<D, BS>::NW)) void decode_kernel(DecodeParams p) {
  using Sh = DecodeShape<D, BS>;
  constexpr int LPR = Sh::LPR, RPL = Sh::RPL, LPB = Sh::LPB, BPS = Sh::BPS,
                NL = Sh::NL, NW = Sh::NW;
  constexpr bool SUB = Sh::SUB;
  __shared__ float s_acc[NW][GH][D];
  __shared__ float s_m[NW][GH], s_l[NW][GH];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int HG = p.num_q_heads / GH;
  int idx = blockIdx.x;
  const int hg = idx % HG;
  idx /= HG;
  const int slot = idx % p.num_seqs;
  const int s = p.has_order ? p.order[slot] : slot;
  const int part = idx / p.num_seqs;
  const int h0 = hg * GH;
  const size_t row0 = (size_t)s * p.num_q_heads + h0;  // first output row

  // The sequence length, the partition's block ids (lane j: entry j, read
  // from a table index clamped into the row, so the read needs no length)
  // and the query rows are loaded together, before any of them is used:
  // one memory latency before the first K/V load instead of three.
  // Blocks that hold whole wave-wide loads allow partitions of up to 256
  // blocks (4 ids per lane); smaller blocks 64 (one id per lane, fetched
  // by the lanes that need it).
  const int part_blocks = p.part_tokens / BS;
  const int blk0 = part * part_blocks;  // < max_blocks_per_seq: part < num_parts
  const int32_t *trow = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  PartitionIds<SUB ? 1 : kIdsPerLane> ids;
  ids.issue(trow, blk0, p.max_blocks_per_seq, lane);
  const int L = p.seq_lens[s];
  const int col = lane % LPR;   // 16-byte column within a token row
  const int rrow = lane / LPR;  // token row within one wave-wide load
  h8_t qv[GH];
#pragma unroll
  for (int g = 0; g < GH; ++g)
    qv[g] = as_h8(ld16(p.q + (row0 + g) * D + col * 8));

  if (!(L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS)) {
    if (part == 0)
      for (int i = threadIdx.x; i < GH * D; i += blockDim.x)
        p.out[row0 * D + i] = __builtin_nanf("");
    return;
  }
  const int np_row = cdiv(L, p.part_tokens);
  if (part >= np_row) return;

  const int kvh = h0 / p.group;
  const int nblk = cdiv(L, BS);
  const int blk1 = min(blk0 + part_blocks, nblk);
  // A wave step may overhang the partition's last block; those zero-filled
  // rows must not enter the softmax.
  const int tok_end = min(L, blk1 * BS);

  // An id outside the pool poisons the whole sequence (every wave sees the
  // same slice).
  const bool bad = __any(ids.settle(blk1 - blk0, p.num_blocks, lane));

  float m[GH], lsum[GH], acc[GH][8];
#pragma unroll
  for (int g = 0; g < GH; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[g][k] = 0.f;
  }
  const size_t head_elems = (size_t)BS * D;
  const uint4 zero = make_uint4(0, 0, 0, 0);

  for (int b = blk0 + wave * BPS; b < blk1; b += NW * BPS) {
    uint4 kr[NL], vr[NL];
    if constexpr (!SUB) {
#pragma unroll
      for (int c = 0; c < BPS; ++c) {
        const int bb = b + c;
        const bool in = bb < blk1;
        const int phys = ids.get(in ? bb - blk0 : 0);
        const size_t base =
            ((size_t)phys * p.num_kv_heads + kvh) * head_elems + rrow * D + col * 8;
#pragma unroll
        for (int j = 0; j < LPB; ++j) {
          if (in) {
            kr[c * LPB + j] = ld16_nt(p.k_cache + base + (size_t)j * RPL * D);
            vr[c * LPB + j] = ld16_nt(p.v_cache + base + (size_t)j * RPL * D);
          } else {
            kr[c * LPB + j] = zero;
            vr[c * LPB + j] = zero;
          }
        }
      }
    } else {
      // Per-lane block ids from the lanes that hold them; a token past the
      // partition reads entry 0's block (in bounds) and is masked below.
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int tok = b * BS + i * RPL + rrow;
        const int bl = tok / BS - blk0;
        const int phys = __shfl(ids.v[0], bl < blk1 - blk0 ? bl : 0, kWave);
        const size_t off = ((size_t)phys * p.num_kv_heads + kvh) * head_elems +
                           (size_t)(tok % BS) * D + col * 8;
        kr[i] = ld16_nt(p.k_cache + off);
        vr[i] = ld16_nt(p.v_cache + off);
      }
    }
#pragma unroll
    for (int g = 0; g < GH; ++g) {
      float sc[NL];
      float cmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int tok = b * BS + i * RPL + rrow;
        const float d = group_sum<LPR>(dot8(qv[g], as_h8(kr[i]), 0.f));
        sc[i] = tok < tok_end ? d * p.scale_log2e : -INFINITY;
        cmax = fmaxf(cmax, sc[i]);
      }
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) cmax = xor_max(cmax, off);
      // the step's first token is always valid, so mnew is finite
      const float mnew = fmaxf(m[g], cmax);
      const float alpha = fast_exp2(m[g] - mnew);
      lsum[g] *= alpha;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[g][k] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int tok = b * BS + i * RPL + rrow;
        const bool ok = tok < tok_end;
        const float pr = ok ? fast_exp2(sc[i] - mnew) : 0.f;
        const h8_t v = as_h8(ok ? vr[i] : zero);
        lsum[g] += pr;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[g][k] = fmaf(pr, (float)v[k], acc[g][k]);
      }
      m[g] = mnew;
    }
  }

  // Lanes of one row group hold equal sums; add the row groups.
#pragma unroll
  for (int g = 0; g < GH; ++g) {
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
      lsum[g] = xor_sum(lsum[g], off);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[g][k] = xor_sum(acc[g][k], off);
    }
    if (lane < LPR) {
#pragma unroll
      for (int k = 0; k < 8; ++k) s_acc[wave][g][col * 8 + k] = acc[g][k];
    }
    if (lane == 0) {
      s_m[wave][g] = m[g];
      s_l[wave][g] = lsum[g];
    }
  }
  __syncthreads();

  const bool split = np_row > 1;
  for (int i = threadIdx.x; i < GH * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float e = fast_exp2(s_m[w][g] - M);  // an idle wave has m = -inf
      o = fmaf(e, s_acc[w][g][d], o);
      l = fmaf(e, s_l[w][g], l);
    }
    if (bad) o = __builtin_nanf("");
    if (!split) {
      p.out[(row0 + g) * D + d] = o / l;
    } else {
      const size_t pi = (row0 + g) * p.num_parts + part;
      p.ws_o[pi * D + d] = o;
      if (d == 0) {
        p.ws_m[pi] = M;
        p.ws_l[pi] = l;
      }
    }
  }
}

// Decode for 4, 8 or 16 query heads per workgroup (GH) sharing one KV head,
// on the matrix cores.
//
// With 8 query heads sharing every K/V row, the scores of a 32-token step
// are the product of an [8 x D] query block with D x 32 keys, and the output
// update is an [8 x 32] weight block times 32 x D values: dense contractions
// of 8 FLOP per logical K/V byte, past the point where the vector ALUs (no
// packed fp32) keep up with HBM.  Both run here as v_mfma_f32_16x16x32_f16
// tiles with the GH query heads as the 16 columns (4 or 8 heads padded with
// zeros; 16 heads fill them, so one workgroup reads each K/V row for all).
// At 4 heads (4 FLOP per byte) the vector-ALU kernel already falls behind
// HBM, and the same tiles run at the matrix cores' step rate:
// * S^T (16 tokens x 16 heads) = K_tile (16 x D) . Q^T.  Lane l supplies
//   K row l%16, dims 32kk + 8(l/16) .. +7 of k-step kk.  K is loaded with
//   16 lanes per row (whole rows per load instruction, as V) and handed to
//   the operand layout through a wave-private LDS tile: read straight into
//   the operand registers, each load instruction would touch 16 rows in
//   64-byte pieces, which the memory path serves markedly slower.
// * Lane l then holds the scores of head l%16 for tokens 16i + 4(l/16) + r
//   (tile i, r < 4).  Those 8 weights, in that order, are exactly the lane's
//   P^T operand of the next product (contraction index 8(l/16) + j <->
//   token 16(j/4) + 4(l/16) + j%4), so they move nowhere.
// * O^T (D x 16 heads) += V^T (D x 32 tokens) . P^T.  Lane l loads the 16
//   (D = 128) or 8 (D = 64) bytes at dims VD*(l%16) .. of its 8 tokens:
//   each load instruction reads 4 whole rows.  An 8 x 8 (or 4 x 8) register
//   transpose turns them into the V^T operands of VD m-tiles, m-tile mt
//   holding dim VD*(l%16) + mt in row l%16.  Lane l ends with head l%16's
//   output at the contiguous dims 4VD(l/16) .. 4VD(l/16) + 4VD - 1.
// * The fp32 weights enter the PV as an fp16 high part and an fp16 low part
//   (two MFMAs), so the product keeps about 22 bits of each weight, as fp32
//   accumulation on the vector ALUs would.
// * Softmax runs in base 2 with a running maximum that only moves when a
//   head's maximum exceeds it by 2^8; masked tokens are removed by
//   selection.
template <int D, int BS, int GH>
__global__ __launch_bounds__(256) void decode_gqa_mfma_kernel(DecodeParams p) {
  static_assert(GH == 4 || GH == 8 || GH == 16, "4, 8 or 16 query heads per workgroup");
  constexpr int NW = 4;
  constexpr int TOK = 32;        // tokens per wave step: two 16-row tiles
  constexpr int CH = TOK / BS;   // blocks per wave step
  constexpr int KQ = D / 32;     // k-steps of the score product
  constexpr int VD = D / 16;     // dims per lane of a V row; PV m-tiles
  constexpr int SLOTS = D / 8;         // 16-byte chunks of a row
  constexpr int KRPI = kWave / SLOTS;  // K rows per coalesced wave-wide load
  constexpr int KNI = 16 / KRPI;       // K loads per lane per 16-row tile
  static_assert(BS == 8 || BS == 16 || BS == 32, "a 16-row tile in one or two blocks");
  constexpr bool TWO = BS < 16;  // a tile spans two blocks
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  // Wave-private K tile (swizzled); after its last step a wave stores its
  // partial output [GH][D] fp32 in the same place (GH*D*4 <= TOK*SLOTS*16
  // bytes), so the workgroup needs no LDS beyond its K tiles.  The two views
  // are members of one union.
  union WaveTile {
    uint4 k[TOK * SLOTS];
    float o[GH * D];
  };
  __shared__ WaveTile sK[NW];
  static_assert(sizeof(float) * GH * D <= sizeof(uint4) * TOK * SLOTS,
                "partial output fits the K tile");
  __shared__ float s_m[NW][GH], s_l[NW][GH];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int HG = p.num_q_heads / GH;
  int idx = blockIdx.x;
  const int hg = idx % HG;
  idx /= HG;
  const int slot = idx % p.num_seqs;
  const int s = p.has_order ? p.order[slot] : slot;
  const int part = idx / p.num_seqs;
  const int h0 = hg * GH;
  const size_t row0 = (size_t)s * p.num_q_heads + h0;
  const int hc = lane & 15;  // MFMA column (head) / row (token or dim) index
  const int g = lane >> 4;   // contraction group of the lane

  // Length, block ids (clamped table index) and query rows are loaded
  // together, as in decode_kernel.  Q^T operand: head hc, zero for hc >= GH
  // (the address is clamped into the head group).
  // A partition holds up to 256 blocks, 4 ids per lane.
  const int part_blocks = p.part_tokens / BS;
  const int blk0 = part * part_blocks;
  const int32_t *trow = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  PartitionIds<kIdsPerLane> ids;
  ids.issue(trow, blk0, p.max_blocks_per_seq, lane);
  const int L = p.seq_lens[s];
  const uint4 zero = make_uint4(0, 0, 0, 0);
  h8_t qv[KQ];
#pragma unroll
  for (int kk = 0; kk < KQ; ++kk) {
    const uint4 r = ld16(p.q + (row0 + (hc & (GH - 1))) * D + (4 * kk + g) * 8);
    qv[kk] = as_h8(hc < GH ? r : zero);
  }

  if (!(L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS)) {
    if (part == 0)
      for (int i = threadIdx.x; i < GH * D; i += blockDim.x)
        p.out[row0 * D + i] = __builtin_nanf("");
    return;
  }
  const int np_row = cdiv(L, p.part_tokens);
  if (part >= np_row) return;

  const int kvh = h0 / p.group;
  const int nblk = cdiv(L, BS);
  const int blk1 = min(blk0 + part_blocks, nblk);
  const int tok_end = min(L, blk1 * BS);

  const bool bad = __any(ids.settle(blk1 - blk0, p.num_blocks, lane));
  // physical block of the partition's j-th block (j wave-uniform, < nb)
  auto block_id = [&](int j) -> int { return ids.get(j); };

  float m = -INFINITY, lsum = 0.f;  // head hc; the 4 lanes of a head agree on m
  f4_t acc[VD];
#pragma unroll
  for (int mt = 0; mt < VD; ++mt) acc[mt] = f4_t{0.f, 0.f, 0.f, 0.f};
  const size_t head_elems = (size_t)BS * D;
  const float cs = p.scale_log2e;

  const int kcol = lane % SLOTS, krow = lane / SLOTS;  // K load layout
  uint4 *Kw = sK[wave].k;

  // One wave step: 32 tokens starting at block b.  (Issuing each step's loads
  // one step ahead, in a second register buffer, measured no faster: it
  // costs a wave per SIMD.)
  using KRegs = uint4[2][KNI];           // K: tile i, row q*KRPI + krow, chunk kcol
  using VRegs = uint32_t[2][4][VD / 2];  // V: tile i, token 16i + 4g + r of the step
  // VD fp16 of one V row (16 or 8 bytes), or zeros
  // Loads are unconditional and keep what they read: a row outside the
  // partition reads a block of the pool (every settled id is one), and every
  // row past the last valid token -- those included -- has its score
  // replaced by -inf and its V row by zeros in compute_step.  A load under a
  // branch, or a select right after it, would make the compiler wait for
  // that load before issuing the next ones.
  auto load_v = [&](uint32_t (&dst)[VD / 2], const _Float16 *src) {
    if constexpr (VD == 8) {
      const uint4 v = ld16_nt(src);
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    } else {
      const uint2 v = ld8_nt(src);
      dst[0] = v.x; dst[1] = v.y;
    }
  };
  // All K loads of the step are issued before its V loads: the K tile is
  // stored and consumed (scores, softmax) while the V loads are still in
  // flight, and the wait before the K store counts only the K loads.
  auto load_step = [&](int b, KRegs &kr, VRegs &vr) {
    if constexpr (!TWO) {
      bool in[2];
      const _Float16 *kb[2], *vb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // tile i lies in block b + 16i/BS, from its row 16i % BS
        const int bi = (16 * i) / BS;
        in[i] = b + bi < blk1;
        const int phys = block_id(in[i] ? b + bi - blk0 : 0);
        const size_t base = ((size_t)phys * p.num_kv_heads + kvh) * head_elems +
                            (size_t)((16 * i) % BS) * D;
        kb[i] = p.k_cache + base + (size_t)krow * D + 8 * kcol;
        vb[i] = p.v_cache + base + (size_t)(4 * g) * D + VD * hc;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < KNI; ++q)
        kr[i][q] = ld16_nt(kb[i] + (size_t)q * KRPI * D);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) load_v(vr[i][r], vb[i] + (size_t)r * D);
    } else {
      // block size 8: rows 0-7 of tile i in block A = b + 2i, rows 8-15 in
      // block B = b + 2i + 1.  K load q holds rows q*KRPI .. +KRPI-1 (one
      // block); V row 4g + r is in block B for g >= 2.
      bool inA[2], inB[2];
      size_t baseA[2], baseB[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int bA = b + 2 * i, bB = bA + 1;
        inA[i] = bA < blk1;
        inB[i] = bB < blk1;
        const int phA = block_id(inA[i] ? bA - blk0 : 0);
        const int phB = block_id(inB[i] ? bB - blk0 : 0);
        baseA[i] = ((size_t)phA * p.num_kv_heads + kvh) * head_elems;
        baseB[i] = ((size_t)phB * p.num_kv_heads + kvh) * head_elems;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < KNI; ++q) {
          const bool hi = q * KRPI >= BS;
          const size_t off = (hi ? baseB[i] : baseA[i]) +
                             (size_t)((q * KRPI + krow) % BS) * D + 8 * kcol;
          kr[i][q] = ld16_nt(p.k_cache + off);
        }
      const bool vhi = g >= 2;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const _Float16 *vb = p.v_cache + (vhi ? baseB[i] : baseA[i]) + VD * hc;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          load_v(vr[i][r], vb + (size_t)((4 * g + r) % BS) * D);
      }
    }
  };
  auto compute_step = [&](int b, KRegs &kr, VRegs &vr) {
    const int tok0 = b * BS;
    const bool full = tok0 + TOK <= tok_end;
    // K through the wave's LDS tile: stored as loaded (16 lanes per row),
    // read back in the operand layout (4 lanes per row).  Chunk c of row t
    // sits at slot c ^ (t % SLOTS), so both the stores (one row's chunks per
    // 8 lanes) and the reads (8 rows' chunk per 8 lanes) hit distinct banks.
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < KNI; ++q) {
        const int t = 16 * i + q * KRPI + krow;
        Kw[t * SLOTS + (kcol ^ (t & (SLOTS - 1)))] = kr[i][q];
      }
    uint4 ka[2][KQ];  // A operand: row 16i + hc, dims 32kk + 8g .. +7
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) {
        const int t = 16 * i + hc;
        ka[i][kk] = Kw[t * SLOTS + ((4 * kk + g) ^ (t & (SLOTS - 1)))];
      }

    // scores of both tiles, scaled to base 2; masked tokens -> -inf
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f4_t sc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) sc = mfma16x16x32(as_h8(ka[i][kk]), qv[kk], sc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[r] * cs;
        if (!full && tok0 + 16 * i + 4 * g + r >= tok_end) v = -INFINITY;
        x[i][r] = v;
        mx = vmax(mx, v);
      }
    }
    // The step's first token is valid, so every head's maximum is finite.
    mx = max_over_rows(mx);
    if (__any(mx > m + kLazyRescale)) {
      const float mnew = vmax(m, mx);
      const float alpha = fast_exp2(m - mnew);  // 0 while m = -inf
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int mt = 0; mt < VD; ++mt) acc[mt] *= alpha;
    }
    // weights: P^T operand, split into fp16 high and low parts
    h8_t phi, plo;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = fast_exp2(x[i][r] - m);
        lsum += e;
        const _Float16 hi = (_Float16)e;
        phi[4 * i + r] = hi;
        plo[4 * i + r] = (_Float16)(e - (float)hi);
      }
    // masked rows carry weight 0 but may hold NaN: select, never multiply
    if (!full) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tok0 + 16 * i + 4 * g + r >= tok_end)
#pragma unroll
            for (int w = 0; w < VD / 2; ++w) vr[i][r][w] = 0;
    }
    // V^T operands: m-tile mt takes half mt of each of the 8 rows
#pragma unroll
    for (int mt = 0; mt < VD; ++mt) {
      uint32_t w4[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = vr[w / 2][2 * (w % 2)][mt / 2];
        const uint32_t c = vr[w / 2][2 * (w % 2) + 1][mt / 2];
        w4[w] = (mt % 2 == 0) ? ((a & 0xffffu) | (c << 16))
                              : ((a >> 16) | (c & 0xffff0000u));
      }
      const h8_t va = __builtin_bit_cast(h8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
      acc[mt] = mfma16x16x32(va, phi, acc[mt]);
      acc[mt] = mfma16x16x32(va, plo, acc[mt]);
    }
  };

  KRegs kr;
  VRegs vr;
  // The partition's steps are walked from an offset given by the sequence
  // index, so that workgroups running side by side read different blocks of
  // a prefix their sequences share (fewer requests piling onto the same L2
  // lines at once).  The order depends on the sequence alone, so results do
  // not depend on the dispatch order or on where blocks sit in the pool.
  const int nsteps = cdiv(blk1 - blk0, CH);
  const int rot = s % nsteps;
  for (int j = wave; j < nsteps; j += NW) {
    const int b = blk0 + CH * (j + rot < nsteps ? j + rot : j + rot - nsteps);
    load_step(b, kr, vr);
    compute_step(b, kr, vr);
  }

  // the 4 lanes of a head hold sums over different tokens
  lsum = sum_over_rows(lsum);
  // The wave's last K-tile reads come before its partial-output stores into
  // the same LDS: a compiler fence keeps that order in the code, and LDS
  // serves one wave's accesses in issue order.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_wave_barrier();
  if (hc < GH) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int mt = 0; mt < VD; ++mt)
        sK[wave].o[hc * D + VD * (4 * g + r) + mt] = acc[mt][r];
    if (g == 0) {
      s_m[wave][hc] = m;
      s_l[wave][hc] = lsum;
    }
  }
  __syncthreads();

  const bool split = np_row > 1;
  for (int i = threadIdx.x; i < GH * D; i += blockDim.x) {
    const int h = i / D, d = i % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float e = s_m[w][h] > -INFINITY ? fast_exp2(s_m[w][h] - M) : 0.f;
      o = fmaf(e, sK[w].o[h * D + d], o);
      l = fmaf(e, s_l[w][h], l);
    }
    if (bad) o = __builtin_nanf("");
    if (!split) {
      p.out[(row0 + h) * D + d] = o / l;
    } else {
      const size_t pi = (row0 + h) * p.num_parts + part;
      p.ws_o[pi * D + d] = o;
      if (d == 0) {
        p.ws_m[pi] = M;
        p.ws_l[pi] = l;
      }
    }
  }
}

// One thread per (row, 4 dims): 256 / (D/4) rows per workgroup.  A row split
// into at most kMergeFast partitions issues all its workspace loads at once
// (one memory round trip after the length); longer rows take the maximum
// first, then the sums, with each chunk's loads issued together.  Both forms
// add in partition order, so a row's result does not depend on which form
// ran.
constexpr int kMergeFast = 4;
template <int D, int BS>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  constexpr int D4 = D / 4, RPW = 256 / D4;
  const size_t row = (size_t)blockIdx.x * RPW + threadIdx.x / D4;
  const size_t rows = (size_t)p.num_seqs * p.num_q_heads;
  if (row >= rows) return;
  const int s = (int)(row / p.num_q_heads);
  const int d = 4 * ((int)threadIdx.x % D4);
  const int L = p.seq_lens[s];
  if (!(L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS))
    return;  // the partition kernel wrote NaN
  const int np = cdiv(L, p.part_tokens);
  if (np == 1) return;  // written directly by the partition kernel
  const size_t base = row * p.num_parts;
  float M = -INFINITY, l = 0.f;
  f4_t o = f4_t{0.f, 0.f, 0.f, 0.f};
  if (np <= kMergeFast) {
    // a partition index past the row's last is clamped to 0 (in bounds,
    // unused)
    float mj[kMergeFast], lj[kMergeFast];
    f4_t oj[kMergeFast];
#pragma unroll
    for (int j = 0; j < kMergeFast; ++j) {
      const size_t pi = base + (j < np ? j : 0);
      mj[j] = p.ws_m[pi];
      lj[j] = p.ws_l[pi];
      oj[j] = *reinterpret_cast<const f4_t *>(p.ws_o + pi * D + d);
    }
#pragma unroll
    for (int j = 0; j < kMergeFast; ++j)
      if (j < np) M = fmaxf(M, mj[j]);
#pragma unroll
    for (int j = 0; j < kMergeFast; ++j)
      if (j < np) {
        const float e = fast_exp2(mj[j] - M);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = fmaf(e, oj[j][k], o[k]);
        l = fmaf(e, lj[j], l);
      }
  } else {
    // the same two passes, each chunk's loads issued together
    for (int j0 = 0; j0 < np; j0 += 2 * kMergeFast) {
      float mj[2 * kMergeFast];
#pragma unroll
      for (int u = 0; u < 2 * kMergeFast; ++u)
        mj[u] = p.ws_m[base + (j0 + u < np ? j0 + u : 0)];
#pragma unroll
      for (int u = 0; u < 2 * kMergeFast; ++u)
        if (j0 + u < np) M = fmaxf(M, mj[u]);
    }
    for (int j0 = 0; j0 < np; j0 += kMergeFast) {
      float mj[kMergeFast], lj[kMergeFast];
      f4_t oj[kMergeFast];
#pragma unroll
      for (int u = 0; u < kMergeFast; ++u) {
        const size_t pi = base + (j0 + u < np ? j0 + u : 0);
        mj[u] = p.ws_m[pi];
        lj[u] = p.ws_l[pi];
        oj[u] = *reinterpret_cast<const f4_t *>(p.ws_o + pi * D + d);
      }
#pragma unroll
      for (int u = 0; u < kMergeFast; ++u)
        if (j0 + u < np) {
          const float e = fast_exp2(mj[u] - M);
#pragma unroll
          for (int k = 0; k < 4; ++k) o[k] = fmaf(e, oj[u][k], o[k]);
          l = fmaf(e, lj[u], l);
        }
    }
  }
  *reinterpret_cast<f4_t *>(p.out + row * D + d) = o / l;
}

// Batches whose rows may hold more than kMergeFast partitions: one
// workgroup per row.  Thread group j (256 / (D/4) groups of one thread per 4
// dims) combines partitions j, j + groups, ... in registers, a chunk of
// kMergeFast partitions' loads at a time, with the running-maximum rescale;
// the groups' (maximum, sum, output) are then combined through LDS.  A row
// takes two memory round trips after its length instead of one per chunk.
template <int D, int BS>
__global__ __launch_bounds__(256) void decode_merge_wide_kernel(DecodeParams p) {
  constexpr int D4 = D / 4, NG = 256 / D4;
  __shared__ float s_gm[NG], s_gl[NG];
  __shared__ f4_t s_go[NG][D4];
  const size_t row = blockIdx.x;
  const int s = (int)(row / p.num_q_heads);
  const int c = (int)threadIdx.x % D4, grp = (int)threadIdx.x / D4;
  const int L = p.seq_lens[s];
  if (!(L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS))
    return;  // the partition kernel wrote NaN
  const int np = cdiv(L, p.part_tokens);
  if (np == 1) return;  // written directly by the partition kernel
  const size_t base = row * p.num_parts;
  float M = -INFINITY, l = 0.f;
  f4_t o = f4_t{0.f, 0.f, 0.f, 0.f};
  for (int j0 = grp; j0 < np; j0 += NG * kMergeFast) {
    float mj[kMergeFast], lj[kMergeFast];
    f4_t oj[kMergeFast];
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u) {
      const int j = j0 + u * NG;
      const size_t pi = base + (j < np ? j : 0);  // past the last: in bounds, unused
      mj[u] = p.ws_m[pi];
      lj[u] = p.ws_l[pi];
      oj[u] = *reinterpret_cast<const f4_t *>(p.ws_o + pi * D + 4 * c);
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u)
      if (j0 + u * NG < np) cm = fmaxf(cm, mj[u]);
    const float a = fast_exp2(M - cm);  // 0 on the first chunk (M = -inf)
    o *= a;
    l *= a;
#pragma unroll
    for (int u = 0; u < kMergeFast; ++u)
      if (j0 + u * NG < np) {
        const float e = fast_exp2(mj[u] - cm);
        o += e * oj[u];
        l += e * lj[u];
      }
    M = cm;
  }
  // a group with no partition keeps M = -inf, l = 0, o = 0
  if (c == 0) {
    s_gm[grp] = M;
    s_gl[grp] = l;
  }
  s_go[grp][c] = o;
  __syncthreads();
  if (grp != 0) return;
  float Mt = s_gm[0];
#pragma unroll
  for (int k = 1; k < NG; ++k) Mt = fmaxf(Mt, s_gm[k]);
  f4_t ot = f4_t{0.f, 0.f, 0.f, 0.f};
  float lt = 0.f;
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const float e = s_gm[k] > -INFINITY ? fast_exp2(s_gm[k] - Mt) : 0.f;
    ot += e * s_go[k][c];
    lt += e * s_gl[k];
  }
  *reinterpret_cast<f4_t *>(p.out + row * D + 4 * c) = ot * (1.f / lt);
}

template <int D, int BS, int GH>
static hipError_t launch(const DecodeParams &p, hipStream_t stream) {
  const int64_t grid =
      (int64_t)p.num_parts * p.num_seqs * (p.num_q_heads / GH);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  // 4, 8 or 16 heads per workgroup: matrix-core tiles of 16 rows in one or
  // two blocks (block sizes 8, 16 and 32).  Fewer heads per workgroup, and
  // block size 1, take the vector-ALU kernel (at 2 heads both run at the
  // same speed; from 4 heads the vector ALUs fall behind HBM).
  if constexpr (GH >= 4 && BS >= 8)
    decode_gqa_mfma_kernel<D, BS, GH><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(p);
  else
    decode_kernel<D, BS, GH>
        <<<dim3((unsigned)grid), dim3(64 * DecodeShape<D, BS>::NW), 0, stream>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_parts == 1) return e;
  const int64_t rows = (int64_t)p.num_seqs * p.num_q_heads;
  constexpr int RPW = 256 / (D / 4);  // rows per merge workgroup
  if (p.num_parts <= kMergeFast)
    decode_merge_kernel<D, BS><<<dim3((unsigned)((rows + RPW - 1) / RPW)), dim3(256), 0, stream>>>(p);
  else
    decode_merge_wide_kernel<D, BS><<<dim3((unsigned)rows), dim3(256), 0, stream>>>(p);
  return hipGetLastError();
}

template <int D, int BS>
static hipError_t launch_heads(const DecodeParams &p, hipStream_t stream) {
  switch (heads_per_workgroup(p.group, BS)) {
    case 16:
      if constexpr (BS >= 8) return launch<D, BS, 16>(p, stream);
      return hipErrorInvalidValue;
    case 8: return launch<D, BS, 8>(p, stream);
    case 4: return launch<D, BS, 4>(p, stream);
    case 2: return launch<D, BS, 2>(p, stream);
    default: return launch<D, BS, 1>(p, stream);
  }
}

hipError_t launch_decode(const DecodeParams &p, int head_dim, int block_size,
                         hipStream_t stream) {
  if (p.part_tokens <= 0 || p.part_tokens % block_size || p.group <= 0 ||
      p.num_q_heads % p.group ||
      p.part_tokens > max_partition_blocks(block_size) * block_size)
    return hipErrorInvalidValue;
  if (head_dim == 128) {
    switch (block_size) {
      case 1: return launch_heads<128, 1>(p, stream);
      case 8: return launch_heads<128, 8>(p, stream);
      case 16: return launch_heads<128, 16>(p, stream);
      case 32: return launch_heads<128, 32>(p, stream);
    }
  } else if (head_dim == 64) {
    switch (block_size) {
      case 1: return launch_heads<64, 1>(p, stream);
      case 8: return launch_heads<64, 8>(p, stream);
      case 16: return launch_heads<64, 16>(p, stream);
      case 32: return launch_heads<64, 32>(p, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
