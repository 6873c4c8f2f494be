// Paged attention prefill of causal chunks on MFMA.
//
// What is computed ("LLM 推理引擎 Continuous Batching 与 PagedAttention：从
// vLLM 原理到生产级部署实战", §4.3 Chunked Prefill, with the causal rule of
// the prefill phase in §1.1): a chunk of C new tokens sits on a prefix of P
// tokens that is already in paged blocks; query row j of the chunk is token
// P + j of its sequence and attends to keys 0 .. P + j, read through the
// block table exactly as the decode does.
//
// Design for CDNA4 (gfx950, wave64, v_mfma_f32_16x16x32_f16):
// * One workgroup of 4 waves takes a 128-row query tile of one (chunk, head);
//   each wave owns 32 query rows (two 16-column MFMA blocks), so every
//   operand fragment read from LDS feeds two MFMAs.
// * Key/value tiles of 64 tokens go from the paged pool straight into LDS
//   (direct-to-LDS loads, one block id per load instruction, read one tile
//   ahead); two buffers per operand, so the next tile's loads are in flight
//   while the current one is consumed.  K and V stay row-major.
// * Per tile and wave:
//     S^T = K Q^T     A = 16 keys x 32 dims from LDS, B = the wave's query
//                     rows, kept in registers;
//     online softmax  base 2, running max and sum per query row; a row's
//                     values sit in the 4 lanes with the same l % 16, so the
//                     max needs two cross-lane steps; the running max only
//                     moves when a row's maximum exceeds it by 2^8 (the
//                     weights, at most 256, stay exact enough in fp16), so
//                     the O rescale is rare;
//     O^T += V^T P^T  the accumulator layout of S^T is the B-operand layout
//                     of P^T, so the fp16 weights never leave their lanes;
//                     the V^T operand comes from V rows by two transposing
//                     LDS reads (ds_read_b64_tr_b16) per 8 keys.
//   The 16 keys of each S^T block are taken in a permuted order chosen so
//   that lane group g ends up holding 8 consecutive keys of each 32-key
//   step, the keys the V^T operand's transposing reads deliver.
// * Keys above the diagonal are removed by selection in the diagonal tiles
//   only; a wave skips tiles that lie wholly above its rows.  The heaviest
//   query tiles (last in their chunk) are dispatched first.
// * When the query tiles are too few to fill the chip, each one's key range
//   is cut into parts run by different workgroups, merged by a second
//   kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace pkv {

// log2 of the largest softmax weight tolerated before the running maximum is
// moved (weights enter the PV product as fp16)
constexpr float kLazyRescale = 8.f;
// Starting value of the running maximum (log2 units): finite and far below
// any score q.k * scale * log2(e) of fp16 operands.  A row that has not met
// a visible key yet keeps it: masked keys then give exp2(-inf) = 0 and
// rescale factors exp2(floor - m) are 0 (or 1), never inf - inf.  (A part
// of a split key range can start on a tile that hides every key from some
// of a wave's rows.)
constexpr float kMaxFloor = -1e30f;

// LDS layout.  K and V tiles arrive by direct-to-LDS loads: one load
// instruction writes its 64 lanes' 16-byte chunks to 1 KB of consecutive LDS
// (lane l at byte 16 l), and each lane fetches the global chunk that belongs
// at its position.  Tiles are row-major without padding; the 16-byte slot s
// of tile row r sits at chunk r * SL + (s ^ swizzle(r)), SL = D / 8 slots per
// row.  Timed on this chip, a wave's 16-byte LDS reads run at full rate when
// every 8 consecutive lanes touch chunks that differ modulo 16 (256 bytes)
// and every 32 consecutive lanes chunks that differ modulo 32 (512 bytes):
// kswz() gives both for the QK^T operand reads of K rows (16 rows by two
// slots per half-wave), vswz() the best rate measured for the transposing
// reads (ds_read_b64_tr_b16) that give the PV operand from V rows.
template <int SL>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (SL == 16)
    return ((r & 1) ^ ((r >> 4) & 1)) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 3);
  else
    return (((r >> 1) & 1) ^ ((r >> 4) & 1)) | (((r >> 3) & 1) << 2);
}
template <int SL>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (SL == 16)
    return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
  else
    return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
}

#define PKV_AS1 __attribute__((address_space(1)))
#define PKV_AS3 __attribute__((address_space(3)))

// Direct-to-LDS loads of 16 bytes per lane: the global address is a scalar
// base (the block's, the same in every lane) plus the lane's 32-bit byte
// offset, and lane l writes bytes 16 l .. 16 l + 15 above the LDS base in
// M0.  With the block's base in scalar registers, a tile's loads need no
// per-lane 64-bit address arithmetic (mixed step 39.5 -> 38.0 us against a
// full per-lane address).
//
// Written as the instruction itself rather than the compiler builtin: while
// the compiler tracks a direct-to-LDS load in flight, it treats the LDS
// return counter as unordered and waits for every outstanding LDS read
// (lgkmcnt(0)) before each use of one, so the operand reads of the current
// tile lost all overlap with the MFMAs.  Untracked, its waits are partial
// again.  The instruction writes no register, only LDS; every reader of the
// buffer it fills runs after this kernel's explicit wait for all memory
// counters and a barrier.
//
// N consecutive 1 KB chunks of one block with one M0: the instruction's
// immediate offset (k KB for chunk k) is added to both the global address
// gbase + off[k] and the LDS address lds, so chunk k lands at lds + k KB
// and reads gbase + off[k] + k KB (one M0 write per block instead of one
// per load: 0.3-0.9 % faster, bitwise the same).
template <int N>
__device__ __forceinline__ void load_lds16_run(const void *gbase, const unsigned *off, void *lds) {
  const unsigned base = (unsigned)(size_t)(PKV_AS3 void *)lds;
  if constexpr (N == 1) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off[0]), "s"(gbase), "s"(base)
                 : "memory", "m0");
  } else if constexpr (N == 2) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %2\n\t"
                 "global_load_lds_dwordx4 %1, %2 offset:1024"
                 :
                 : "v"(off[0]), "v"(off[1]), "s"(gbase), "s"(base)
                 : "memory", "m0");
  } else {
    static_assert(N == 4, "runs of 1, 2 or 4 chunks");
    asm volatile("s_mov_b32 m0, %5\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %4\n\t"
                 "global_load_lds_dwordx4 %1, %4 offset:1024\n\t"
                 "global_load_lds_dwordx4 %2, %4 offset:2048\n\t"
                 "global_load_lds_dwordx4 %3, %4 offset:3072"
                 :
                 : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(gbase), "s"(base)
                 : "memory", "m0");
  }
}

// Maxima over the 4 lanes of each column (l, l + 16, l + 32, l + 48) of two
// values at once: a swap of the halves between the two registers leaves the
// first value's half-maxima in lanes 0-31 and the second's in lanes 32-63,
// one swap of 16-lane rows finishes both, and a last swap of the halves
// gives each register its own maximum in every lane.
__device__ __forceinline__ void max_over_rows2(float &x, float &y) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                  false, false);
  const float r = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned ru = __float_as_uint(r);
  const auto b = __builtin_amdgcn_permlane16_swap(ru, ru, false, false);
  const unsigned s = __float_as_uint(vmax(__uint_as_float(b[0]), __uint_as_float(b[1])));
  const auto c = __builtin_amdgcn_permlane32_swap(s, s, false, false);
  x = __uint_as_float(c[0]);
  y = __uint_as_float(c[1]);
}

// A tile buffer index known at compile time.
template <int B>
struct Buf {
  static constexpr int value = B;
};

typedef short s4_t __attribute__((ext_vector_type(4)));
// Transposing LDS read: within each 16-lane group, lane j receives element
// j % 4 of the four 8-byte chunks addressed by lanes j / 4 + 4 k, k = 0..3.
__device__ __forceinline__ h4_t ld_tr16(const _Float16 *lds) {
  const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_AS3 s4_t *)(lds));
  return __builtin_bit_cast(h4_t, v);
}

template <int D, int BS>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p,
                                                         int num_qtiles) {
  constexpr int BM = 128, BN = 64, WROWS = 32;
  constexpr int KS = D / 32;   // MFMA steps over the head dimension (QK)
  constexpr int DT = D / 16;   // 16-row blocks of O^T (PV)
  constexpr int SL = D / 8;    // 16-byte slots of a row
  constexpr int RPI = 64 / SL; // tile rows one load instruction fills
  constexpr int NI = 16 / RPI; // load instructions per wave, tile and operand
  // ids of distinct blocks among one wave's 16 tile rows
  constexpr int NBW = BS >= 16 ? 1 : 16 / BS;
  static_assert(BS % RPI == 0, "a load instruction's rows share a block");
  // Two buffers of each tile, as separate variables: every access names its
  // buffer at compile time (the key-tile loop is unrolled by two), so the
  // compiler can tell the reads of one buffer from the direct-to-LDS loads
  // in flight into the other and need not wait for those loads first.
  __shared__ __attribute__((aligned(16))) _Float16 sK0[BN * D], sK1[BN * D];
  __shared__ __attribute__((aligned(16))) _Float16 sV0[BN * D], sV1[BN * D];
  auto kbuf = [&](auto b) -> _Float16 * {
    if constexpr (decltype(b)::value == 0) return sK0; else return sK1;
  };
  auto vbuf = [&](auto b) -> _Float16 * {
    if constexpr (decltype(b)::value == 0) return sV0; else return sV1;
  };
  __shared__ int sBad;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  int idx = blockIdx.x;
  const int h = idx % p.num_q_heads;
  idx /= p.num_q_heads;
  const int c = idx % p.num_chunks;
  idx /= p.num_chunks;
  const int sp = idx % p.num_splits;  // part of the key range
  const int qt = num_qtiles - 1 - idx / p.num_splits;
  const int q_begin = p.cu_q_lens[c], q_end = p.cu_q_lens[c + 1];
  if (q_begin < 0 || q_end > p.total_q || q_end < q_begin) return;
  const int qlen = q_end - q_begin;
  const int row0 = qt * BM;
  if (row0 >= qlen) return;
  const int L = p.seq_lens[c];
  const int P = L - qlen;
  const int Hq = p.num_q_heads;

  if (!(P >= 0 && L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS)) {
    if (sp != 0) return;
    for (int i = tid; i < BM * D; i += 256) {
      const int r = row0 + i / D;
      if (r < qlen)
        p.out[((size_t)(q_begin + r) * Hq + h) * D + i % D] = __builtin_nanf("");
    }
    return;
  }

  const int g = lane >> 4;   // contraction group of this lane
  const int lc = lane & 15;  // row / column index of this lane
  const int wq0 = row0 + wave * WROWS;  // first query row of this wave
  const int kvh = h / p.group;
  const int kv_end = P + min(row0 + BM, qlen);
  const int ntiles = cdiv(kv_end, BN);
  // this workgroup's part of the key tiles: [t_lo, t_hi)
  const int nparts = min(p.num_splits, cdiv(ntiles, p.split_tiles));
  if (sp >= nparts) return;
  const int t_lo = sp * ntiles / nparts, t_hi = (sp + 1) * ntiles / nparts;
  const int32_t *trow = p.block_tables + (size_t)c * p.max_blocks_per_seq;

  // Tile loader.  Wave w fills tile rows 16 w .. 16 w + 15 of K and of V
  // with NI load instructions each; lane l of instruction j fills LDS chunk
  // (NI w + j) * 64 + l, i.e. row 16 w + RPI j + l / SL, LDS slot l % SL,
  // which holds the row's global slot (l % SL) ^ swizzle(row).  The rows of
  // one instruction lie in one block (tile starts are multiples of BS or of
  // 64), so its block id is the same in every lane: read with a scalar load
  // one tile ahead, from a table index clamped to the last live key (always
  // a valid entry), and only its base address differs between tiles.  An id
  // outside the pool reads block 0 instead and sets a flag, gathered once at
  // the end.  V rows of keys at or past the sequence length (tail slots of
  // the last block, or a clamped block) are zeroed once they have landed:
  // their weights are 0, and 0 times a non-finite value would not be.
  // Load instructions of one block (JPB) share one M0 and take their
  // chunk's KB offset from the instruction.
  constexpr int JPB = (BS / RPI) < NI ? (BS / RPI) : NI;
  // the lane's byte offset in its block, less its load's immediate offset
  unsigned koff[NI], voff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r = 16 * wave + RPI * j + lane / SL;
    const int sl = lane % SL;
    const int kr = r % BS;  // row within its block
    koff[j] = (kr * D + 8 * (sl ^ kswz<SL>(r))) * 2 - 1024 * (j % JPB);
    voff[j] = (kr * D + 8 * (sl ^ vswz<SL>(r))) * 2 - 1024 * (j % JPB);
  }
  const size_t head_elems = (size_t)BS * D;
  auto tile_ids = [&](int t, int *ids) {
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
      const int key = uniform(min(t * BN + 16 * wave + BS * u, L - 1));
      ids[u] = trow[key / BS];
    }
  };
  bool bad = false;  // a block id outside the pool was met
  auto issue_tile = [&](auto buf, const int *ids) {
    size_t base[NBW];
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
      const int ph = uniform(ids[u]);
      const bool oob = ph < 0 || ph >= p.num_blocks;
      bad |= oob;
      base[u] = ((size_t)(oob ? 0 : ph) * p.num_kv_heads + kvh) * head_elems;
    }
#pragma unroll
    for (int j = 0; j < NI; j += JPB) {
      const int u = (RPI * j) / BS;
      load_lds16_run<JPB>(p.k_cache + base[u], &koff[j], kbuf(buf) + (NI * wave + j) * 512);
      load_lds16_run<JPB>(p.v_cache + base[u], &voff[j], vbuf(buf) + (NI * wave + j) * 512);
    }
  };
  // after this wave's loads of tile t have landed
  auto zero_tail = [&](int t, auto buf) {
    if (t * BN + 16 * wave + 15 >= L) {
      const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        if (t * BN + 16 * wave + RPI * j + lane / SL >= L)
          st16(vbuf(buf) + ((NI * wave + j) * 64 + lane) * 8, zero);
    }
  };

  f4_t o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    o[dt][0] = o[dt][1] = f4_t{0.f, 0.f, 0.f, 0.f};
  float m[2] = {kMaxFloor, kMaxFloor};
  // Row sums of the softmax weights come out of the matrix pipe: an all-ones
  // V^T block beside the DT blocks of PV gives sum_k P^T[k][q] in every row
  // of its accumulator, in the lanes that hold column q (no vector adds, no
  // cross-lane sum at the end).
  f4_t lacc[2] = {f4_t{0.f, 0.f, 0.f, 0.f}, f4_t{0.f, 0.f, 0.f, 0.f}};
  h8_t ones;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones[j] = (_Float16)1.f;

  if (tid == 0) sBad = 0;
  // Prologue: the block ids of tiles t_lo and t_lo + 1, then the query rows
  // (issued while the ids are in flight), then tile t_lo's loads.
  int ids[NBW], ids_next[NBW];
  tile_ids(t_lo, ids);
  tile_ids(t_lo + 1, ids_next);
  // The wave's query rows as B operands: column lc of block qb, dims of
  // slot KS*g + kk (8 per slot).  Rows past the chunk load its last row
  // (unconditional loads, nothing waits inside a branch); their results are
  // never stored.
  h8_t qf[KS][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = min(wq0 + 16 * qb + lc, qlen - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qf[kk][qb] = as_h8(ld16(p.q + ((size_t)(q_begin + qr) * Hq + h) * D + 8 * (KS * g + kk)));
  }
  issue_tile(Buf<0>{}, ids);
  __builtin_amdgcn_s_waitcnt(0);
  zero_tail(t_lo, Buf<0>{});
  __syncthreads();

  // Per-lane parts of the LDS operand addresses (in fp16 elements).
  // K: A row lc of block mm is key 32*(mm/2) + 8*(lc/4) + 4*(mm%2) + lc%4;
  // its swizzle depends on lc only.
  const int kx = kswz<SL>(8 * (lc >> 2) + (lc & 3));
  const int krow_lane = 8 * (lc >> 2) + (lc & 3);
  // V (transposing reads): lane lc of group g addresses key row
  // 32 ks + 8 g + 4 hh + lc / 4, dims 16 dt + 4 (lc % 4); the row's swizzle
  // depends on lc and g only.
  const int vrow_lane = 8 * g + (lc >> 2);
  const int vx = vswz<SL>(vrow_lane);

  // The wave computes nothing when all its rows lie past the chunk.
  const bool wave_live = wq0 < qlen;
  // One key tile; buffer `buf` holds it, the other receives the next tile.
  auto step = [&](auto buf, int kt) {
    constexpr Buf<1 - decltype(buf)::value> next{};
    const int kbase = kt * BN;
    // the next tile's loads into the other buffer (its last readers passed
    // the barrier that ended the previous step), then the ids of the tile
    // after it
    if (kt + 1 < t_hi) {
      issue_tile(next, ids_next);
      tile_ids(kt + 2, ids_next);
    }
    // skip a tile that lies wholly above this wave's diagonal
    if (wave_live && kbase <= P + wq0 + WROWS - 1) {
      const _Float16 *Kt = kbuf(buf);
      const _Float16 *Vt = vbuf(buf);
      // S^T: the head-dimension step is the outer loop, so the eight
      // accumulators (4 key blocks x 2 query blocks) are independent and
      // back-to-back MFMAs never wait on each other; each step's four K
      // fragments are read one step ahead.
      f4_t st[4][2];
      h8_t fa[2][4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) st[mm][0] = st[mm][1] = f4_t{0.f, 0.f, 0.f, 0.f};
      auto read_k = [&](int kk, h8_t *dst) {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const int r = 32 * (mm >> 1) + 4 * (mm & 1) + krow_lane;
          dst[mm] = as_h8(ld16(&Kt[(r * SL + ((KS * g + kk) ^ kx)) * 8]));
        }
      };
      // Scheduling barriers keep that order: under register pressure the
      // scheduler would sink each read next to its MFMA, and every read's
      // LDS latency would land on the tile's chain.
      read_k(0, fa[0]);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) read_k(kk + 1, fa[(kk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          st[mm][0] = mfma16x16x32(fa[kk & 1][mm], qf[kk][0], st[mm][0]);
          st[mm][1] = mfma16x16x32(fa[kk & 1][mm], qf[kk][1], st[mm][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // lane holds keys kbase + 32*(mm/2) + 8g + 4*(mm%2) + r of column lc
      if (kbase + BN - 1 > P + wq0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int qpos = P + wq0 + 16 * qb + lc;
#pragma unroll
          for (int mm = 0; mm < 4; ++mm)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int kpos = kbase + 32 * (mm >> 1) + 8 * g + 4 * (mm & 1) + r;
              if (kpos > qpos) st[mm][qb][r] = -INFINITY;
            }
        }
      }
      // raw scores; the scale (> 0) is applied inside the exponent.  The
      // lane's 16 scores of each row, two at a time into a 3-way max.
      float tm[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float tmax = st[0][qb][0];
#pragma unroll
        for (int i = 1; i < 15; i += 2)
          tmax = vmax3(tmax, st[i >> 2][qb][i & 3], st[(i + 1) >> 2][qb][(i + 1) & 3]);
        tm[qb] = vmax(tmax, st[3][qb][3]);
      }
      max_over_rows2(tm[0], tm[1]);
      tm[0] *= p.scale_log2e;
      tm[1] *= p.scale_log2e;
      // Lazy rescaling: the running maximum m only moves when some row's
      // maximum exceeds it by more than 2^8, so weights stay below 256
      // (exact enough in fp16) and the O rescale is rare; one branch serves
      // both query blocks.  m starts at a finite floor, so exp2(-inf) = 0
      // removes masked keys also in rows that have not met a visible key yet.
      if (__any(tm[0] > m[0] + kLazyRescale || tm[1] > m[1] + kLazyRescale)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float mnew = fmaxf(m[qb], tm[qb]);
          const float alpha = fast_exp2(m[qb] - mnew);
          m[qb] = mnew;
          lacc[qb] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][qb] *= alpha;
        }
      }
      h8_t pb[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float nm = -m[qb];
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = fast_exp2(fmaf(st[mm][qb][r], p.scale_log2e, nm));
            pb[mm >> 1][qb][4 * (mm & 1) + r] = (_Float16)e;
          }
        }
      }
      // O^T[d][q] += sum_k V^T[d][k] P^T[k][q]; slot j of lane group g is key
      // 32ks + 8g + j on both sides.  Step i = (ks, dt); its V^T fragment
      // (two transposing reads, keys +0..3 and +4..7) is read NFB steps
      // ahead.
      constexpr int NFB = 2;
      auto read_v = [&](int i) {
        const int ks = i / DT, dt = i % DT;
        const int r0 = 32 * ks + vrow_lane;  // + 4 for the second half
        const int slot = (2 * dt + ((lc >> 1) & 1)) ^ vx;
        const int e0 = (r0 * SL + slot) * 8 + 4 * (lc & 1);
        const h4_t lo = ld_tr16(&Vt[e0]);
        const h4_t hi = ld_tr16(&Vt[e0 + 4 * SL * 8]);
        return h8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      h8_t fb[NFB];
#pragma unroll
      for (int i = 0; i < NFB; ++i) fb[i] = read_v(i);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        const h8_t a = fb[i % NFB];
        if (i + NFB < 2 * DT) fb[i % NFB] = read_v(i + NFB);
        __builtin_amdgcn_sched_barrier(0);  // the reads stay NFB steps ahead
        o[i % DT][0] = mfma16x16x32(a, pb[i / DT][0], o[i % DT][0]);
        o[i % DT][1] = mfma16x16x32(a, pb[i / DT][1], o[i % DT][1]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        lacc[0] = mfma16x16x32(ones, pb[ks][0], lacc[0]);
        lacc[1] = mfma16x16x32(ones, pb[ks][1], lacc[1]);
      }
    }
    // the next tile has landed (this wave's part), its dead V rows are
    // cleared, then every wave's part is visible after the barrier
    __builtin_amdgcn_s_waitcnt(0);
    if (kt + 1 < t_hi) zero_tail(kt + 1, next);
    __syncthreads();
  };
  for (int kt = t_lo; kt < t_hi; kt += 2) {
    step(Buf<0>{}, kt);
    if (kt + 1 < t_hi) step(Buf<1>{}, kt + 1);
  }

  if (bad) sBad = 1;
  __syncthreads();
  const bool any_bad = sBad != 0;
  const f4_t nan4 = f4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                         __builtin_nanf("")};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = lacc[qb][0];  // every row of the ones block holds the sum
    const int qr = wq0 + 16 * qb + lc;
    if (qr >= qlen) continue;
    const size_t row = (size_t)(q_begin + qr) * Hq + h;
    if (nparts == 1) {
      float *orow = p.out + row * D;
      const float inv = 1.f / lt;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f4_t *>(orow + 16 * dt + 4 * g) = any_bad ? nan4 : o[dt][qb] * inv;
    } else {
      // partial of this part: unnormalised output, row maximum, row sum
      const size_t prow = (size_t)sp * p.total_q * Hq + row;
      float *orow = p.ws_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f4_t *>(orow + 16 * dt + 4 * g) = any_bad ? nan4 : o[dt][qb];
      if (g == 0) {
        p.ws_m[prow] = m[qb];
        p.ws_l[prow] = lt;
      }
    }
  }
}

// Combines the parts of query tiles whose key range was split: per row,
// M = max_i m_i, out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i (the
// running-maximum rescale of the softmax recurrence, applied across parts).
// One thread per (row, 4 dims), in one pass: a workgroup takes
// kMergeRows = 256 / (D/4) consecutive rows of one (query tile, chunk,
// head), so a query tile is 128 / kMergeRows workgroups.
template <int D, int BS>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p, int num_qtiles) {
  constexpr int BM = 128, BN = 64, D4 = D / 4, kMergeRows = 256 / D4;
  constexpr int kSubs = BM / kMergeRows;
  int idx = blockIdx.x;
  const int sub = idx % kSubs;
  idx /= kSubs;
  const int Hq = p.num_q_heads;
  const int h = idx % Hq;
  idx /= Hq;
  const int c = idx % p.num_chunks;
  const int qt = num_qtiles - 1 - idx / p.num_chunks;
  const int q_begin = p.cu_q_lens[c], q_end = p.cu_q_lens[c + 1];
  if (q_begin < 0 || q_end > p.total_q || q_end < q_begin) return;
  const int qlen = q_end - q_begin;
  const int row0 = qt * BM;
  const int qr = row0 + sub * kMergeRows + (int)threadIdx.x / D4;
  if (qr >= qlen) return;
  const int L = p.seq_lens[c];
  const int P = L - qlen;
  if (!(P >= 0 && L >= 1 && L <= p.max_seq_len && L <= p.max_blocks_per_seq * BS))
    return;  // the partition kernel wrote NaN
  const int ntiles = cdiv(P + min(row0 + BM, qlen), BN);
  const int nparts = min(p.num_splits, cdiv(ntiles, p.split_tiles));
  if (nparts == 1) return;  // written directly
  const size_t plane = (size_t)p.total_q * Hq;  // rows of one part
  const size_t row = (size_t)(q_begin + qr) * Hq + h;
  const int d = 4 * ((int)threadIdx.x % D4);
  // kChunk parts at a time in one online pass, all loads of a chunk issued
  // together (a part index past the last is clamped to part 0, its values
  // unused); part 0 holds key 0, which every row sees, so m_0 is a score.
  constexpr int kChunk = 4;
  float M = -INFINITY, l = 0.f;
  f4_t o = f4_t{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nparts; j0 += kChunk) {
    float mj[kChunk], lj[kChunk];
    f4_t oj[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const size_t pr = (size_t)(j0 + u < nparts ? j0 + u : 0) * plane + row;
      mj[u] = p.ws_m[pr];
      lj[u] = p.ws_l[pr];
      oj[u] = *reinterpret_cast<const f4_t *>(p.ws_o + pr * D + d);
    }
    float cm = M;
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (j0 + u < nparts) cm = fmaxf(cm, mj[u]);
    const float a = fast_exp2(M - cm);  // 0 on the first chunk (M = -inf)
    o *= a;
    l *= a;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (j0 + u < nparts) {
        const float e = fast_exp2(mj[u] - cm);
        o += e * oj[u];
        l += e * lj[u];
      }
    }
    M = cm;
  }
  *reinterpret_cast<f4_t *>(p.out + row * D + d) = o * (1.f / l);
}

template <int D, int BS>
static hipError_t launch(const PrefillParams &p, int max_q_len,
                         hipStream_t stream) {
  if (p.num_chunks == 0 || max_q_len == 0) return hipSuccess;
  const int qtiles = cdiv(max_q_len, 128);
  const int64_t tiles = (int64_t)qtiles * p.num_chunks * p.num_q_heads;
  const int64_t grid = tiles * p.num_splits;
  constexpr int kMergeSubs = 128 / (256 / (D / 4));  // merge workgroups per query tile
  if (grid > 0x7fffffff || tiles * kMergeSubs > 0x7fffffff || p.num_splits < 1 ||
      p.split_tiles < 1)
    return hipErrorInvalidValue;
  prefill_kernel<D, BS><<<dim3((unsigned)grid), dim3(256), 0, stream>>>(p, qtiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_splits == 1) return e;
  prefill_merge_kernel<D, BS>
      <<<dim3((unsigned)(tiles * kMergeSubs)), dim3(256), 0, stream>>>(p, qtiles);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams &p, int head_dim, int block_size,
                          int max_q_len, hipStream_t stream) {
  if (head_dim == 128 && block_size == 8) return launch<128, 8>(p, max_q_len, stream);
  if (head_dim == 128 && block_size == 16) return launch<128, 16>(p, max_q_len, stream);
  if (head_dim == 128 && block_size == 32) return launch<128, 32>(p, max_q_len, stream);
  if (head_dim == 64 && block_size == 8) return launch<64, 8>(p, max_q_len, stream);
  if (head_dim == 64 && block_size == 16) return launch<64, 16>(p, max_q_len, stream);
  if (head_dim == 64 && block_size == 32) return launch<64, 32>(p, max_q_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
