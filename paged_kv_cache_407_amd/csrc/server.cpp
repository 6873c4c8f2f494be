// Native step executor for continuous batching: one scheduler step planned
// into pinned staging memory and the step's kernels enqueued, with no
// per-step allocation ("LLM 推理引擎 Continuous Batching 与 PagedAttention",
// §2.2: each forward step runs the recomposed batch, prefill chunks and
// decode rows together).
//
// pkv_server_plan: waits until the staging buffer it is about to reuse has
// been copied (two buffers in turn), runs pkv_sched_step into it, and
// enqueues its host-to-device copy on the executor's own copy stream, after
// the kernels of the step that last read that device buffer.
// pkv_server_execute: makes the caller's stream wait for the plan's copy,
// then enqueues pkv_kv_append of the step's new rows, the prefill of its
// chunks and the decode of its decode rows, reading the plan from the
// device copy.  The copy of the next step's plan thus runs beside this
// step's kernels instead of between two steps.
// Staging and the attention workspace are allocated once, when the server
// is created; the caller owns the pools, the new rows and the outputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "pkv.h"

struct pkv_server {
  pkv_scheduler *sched;
  void *k_cache, *v_cache;
  int32_t Hq, Hkv, D, bs, NB, pad, B, T, MB, max_seq_len;
  float scale;
  // int32 staging layout: cu_q_lens [B+1] | prefill_tables [B*MB] |
  // prefill_lens [B] | decode_tables [B*MB] | decode_lens [B] | slots [T+B]
  size_t o_cu, o_pt, o_pl, o_dt, o_dl, o_sl, n_ints;
  int32_t *host[2] = {nullptr, nullptr};
  int32_t *dev[2] = {nullptr, nullptr};
  hipEvent_t copied[2] = {nullptr, nullptr};   // plan i is on the device
  hipEvent_t consumed[2] = {nullptr, nullptr}; // the kernels reading dev[i] are done
  bool pending[2] = {false, false};
  bool in_use[2] = {false, false};             // consumed[i] was recorded
  hipStream_t copy_stream = nullptr;
  int64_t *ids = nullptr;  // [4][B]: prefill, decode, finished, preempted
  void *ws = nullptr;
  size_t ws_bytes = 0;
  std::vector<int32_t> order;  // decode dispatch order of the current step
  int cur = 1;  // staging buffer of the last plan
  pkv_step_plan plan{};
  bool planned = false;

  void release() {
    for (int i = 0; i < 2; ++i) {
      if (copied[i]) (void)hipEventSynchronize(copied[i]);
      if (consumed[i]) (void)hipEventSynchronize(consumed[i]);
    }
    if (copy_stream) (void)hipStreamSynchronize(copy_stream);
    for (int i = 0; i < 2; ++i) {
      if (host[i]) (void)hipHostFree(host[i]);
      if (dev[i]) (void)hipFree(dev[i]);
      if (copied[i]) (void)hipEventDestroy(copied[i]);
      if (consumed[i]) (void)hipEventDestroy(consumed[i]);
    }
    if (copy_stream) (void)hipStreamDestroy(copy_stream);
    if (ws) (void)hipFree(ws);
    delete[] ids;
  }
};

extern "C" {

pkv_server *pkv_server_create(pkv_scheduler *sched, pkv_block_manager *bm, void *k_cache,
                              void *v_cache, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t num_blocks, int32_t pad_block,
                              int32_t max_batch_size, int32_t max_num_tokens,
                              int32_t max_seq_len, float scale) {
  if (!sched || !bm || !k_cache || !v_cache || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || head_dim <= 0 || num_blocks <= 0 || max_batch_size <= 0 ||
      max_num_tokens <= 0 || max_seq_len <= 0 || !(scale > 0.f))
    return nullptr;
  pkv_server *s = new (std::nothrow) pkv_server();
  if (!s) return nullptr;
  s->sched = sched;
  s->k_cache = k_cache;
  s->v_cache = v_cache;
  s->Hq = num_q_heads;
  s->Hkv = num_kv_heads;
  s->D = head_dim;
  s->bs = pkv_bm_block_size(bm);
  s->NB = num_blocks;
  s->pad = pad_block;
  s->B = max_batch_size;
  s->T = max_num_tokens;
  s->max_seq_len = max_seq_len;
  s->MB = (max_seq_len + s->bs - 1) / s->bs;
  s->scale = scale;
  const size_t B = s->B, MB = s->MB;
  s->o_cu = 0;
  s->o_pt = s->o_cu + B + 1;
  s->o_pl = s->o_pt + B * MB;
  s->o_dt = s->o_pl + B;
  s->o_dl = s->o_dt + B * MB;
  s->o_sl = s->o_dl + B;
  s->n_ints = s->o_sl + s->T + B;
  // One workspace serves the step's prefill and decode, which run in turn
  // on one stream.  Decode: the smallest partition the library picks.
  // Prefill: a single chunk of t tokens is split at least as far as any
  // batch of t tokens, and within one 128-row tile count the size grows
  // with t, so the largest need is at a multiple of 128 or at T.
  const int32_t min_part = std::min(256, 64 * s->bs) / s->bs * s->bs;
  s->ws_bytes = pkv_decode_workspace_size(s->B, s->Hq, s->Hkv, s->D, s->bs, max_seq_len,
                                          min_part);
  for (int32_t t = std::min(128, s->T);; t = std::min(t + 128, s->T)) {
    s->ws_bytes = std::max(
        s->ws_bytes, pkv_prefill_workspace_size(1, t, t, s->Hq, s->D, max_seq_len));
    if (t == s->T) break;
  }
  bool ok = (s->ids = new (std::nothrow) int64_t[4 * B]) != nullptr;
  for (int i = 0; i < 2 && ok; ++i)
    ok = hipHostMalloc((void **)&s->host[i], s->n_ints * 4, hipHostMallocDefault) ==
             hipSuccess &&
         hipMalloc((void **)&s->dev[i], s->n_ints * 4) == hipSuccess &&
         hipEventCreateWithFlags(&s->copied[i], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&s->consumed[i], hipEventDisableTiming) == hipSuccess;
  // default priority, like every stream here
  ok = ok && hipStreamCreateWithFlags(&s->copy_stream, hipStreamNonBlocking) == hipSuccess;
  ok = ok && (s->ws_bytes == 0 || hipMalloc(&s->ws, s->ws_bytes) == hipSuccess);
  if (!ok) {
    (void)hipGetLastError();
    s->release();
    delete s;
    return nullptr;
  }
  return s;
}

void pkv_server_destroy(pkv_server *s) {
  if (!s) return;
  s->release();
  delete s;
}

int pkv_server_plan(pkv_server *s, pkv_step_plan *plan, void *stream) {
  if (!s || !plan) return PKV_ERR_INVALID;
  const int i = s->cur ^ 1;
  if (s->pending[i] && hipEventSynchronize(s->copied[i]) != hipSuccess) return PKV_ERR_HIP;
  s->pending[i] = false;
  int32_t *h = s->host[i];
  int64_t *ids = s->ids;
  const int rc = pkv_sched_step(s->sched, s->MB, s->pad, &s->plan, ids, h + s->o_cu,
                                h + s->o_pt, h + s->o_pl, ids + s->B, h + s->o_dt,
                                h + s->o_dl, h + s->o_sl, ids + 2 * s->B, ids + 3 * s->B);
  if (rc != PKV_OK) return rc;
  s->cur = i;
  s->planned = true;
  *plan = s->plan;
  if (s->plan.num_new_tokens == 0) return PKV_OK;
  (void)stream;  // the copy runs on the executor's copy stream
  hipStream_t cs = s->copy_stream;
  if ((s->in_use[i] && hipStreamWaitEvent(cs, s->consumed[i], 0) != hipSuccess) ||
      hipMemcpyAsync(s->dev[i], h, s->n_ints * 4, hipMemcpyHostToDevice, cs) != hipSuccess ||
      hipEventRecord(s->copied[i], cs) != hipSuccess)
    return PKV_ERR_HIP;
  s->pending[i] = true;
  return PKV_OK;
}

int pkv_server_plan_arrays(const pkv_server *s, const int64_t **prefill_ids,
                           const int32_t **cu_q_lens, const int32_t **prefill_lens,
                           const int64_t **decode_ids, const int32_t **decode_lens,
                           const int64_t **finished_ids, const int64_t **preempted_ids) {
  if (!s || !s->planned) return PKV_ERR_INVALID;
  const int32_t *h = s->host[s->cur];
  if (prefill_ids) *prefill_ids = s->ids;
  if (cu_q_lens) *cu_q_lens = h + s->o_cu;
  if (prefill_lens) *prefill_lens = h + s->o_pl;
  if (decode_ids) *decode_ids = s->ids + s->B;
  if (decode_lens) *decode_lens = h + s->o_dl;
  if (finished_ids) *finished_ids = s->ids + 2 * s->B;
  if (preempted_ids) *preempted_ids = s->ids + 3 * s->B;
  return PKV_OK;
}

int pkv_server_execute(pkv_server *s, const void *new_k, const void *new_v, const void *q,
                       float *out_prefill, float *out_decode, void *stream) {
  if (!s || !s->planned) return PKV_ERR_INVALID;
  const pkv_step_plan &p = s->plan;
  if (p.num_new_tokens == 0) return PKV_OK;
  if (!new_k || !new_v || !q || (p.num_prefill && !out_prefill) ||
      (p.num_decode && !out_decode))
    return PKV_ERR_INVALID;
  const int32_t *h = s->host[s->cur];
  const int32_t *d = s->dev[s->cur];
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamWaitEvent(st, s->copied[s->cur], 0) != hipSuccess) return PKV_ERR_HIP;
  int rc = pkv_kv_append(new_k, new_v, s->k_cache, s->v_cache, d + s->o_sl,
                         p.num_new_tokens, s->Hkv, s->D, s->bs, s->NB, stream);
  if (rc != PKV_OK) return rc;
  const size_t qrow = (size_t)s->Hq * s->D * 2;  // bytes of one query row
  if (p.num_prefill) {
    // the step's own bounds: the split of the chunks' key ranges follows them
    int32_t max_q = 0, max_len = 0;
    for (int32_t k = 0; k < p.num_prefill; ++k) {
      max_q = std::max(max_q, h[s->o_cu + k + 1] - h[s->o_cu + k]);
      max_len = std::max(max_len, h[s->o_pl + k]);
    }
    rc = pkv_paged_attention_prefill(out_prefill, q, d + s->o_cu, s->k_cache, s->v_cache,
                                     d + s->o_pt, d + s->o_pl, p.num_prefill,
                                     p.num_prefill_tokens, max_q, s->Hq, s->Hkv, s->D, s->bs,
                                     s->NB, s->MB, max_len, s->scale, s->ws, s->ws_bytes,
                                     stream);
    if (rc != PKV_OK) return rc;
  }
  if (p.num_decode) {
    int32_t max_len = 0;
    for (int32_t k = 0; k < p.num_decode; ++k) max_len = std::max(max_len, h[s->o_dl + k]);
    // dispatch the longest decode rows first (the lengths are on the host)
    s->order.resize(p.num_decode);
    for (int32_t k = 0; k < p.num_decode; ++k) s->order[k] = k;
    const int32_t *dl = h + s->o_dl;
    std::stable_sort(s->order.begin(), s->order.end(),
                     [dl](int32_t a, int32_t b) { return dl[a] > dl[b]; });
    rc = pkv_paged_attention_decode(
        out_decode, (const char *)q + (size_t)p.num_prefill_tokens * qrow, s->k_cache,
        s->v_cache, d + s->o_dt, d + s->o_dl, p.num_decode, s->Hq, s->Hkv, s->D, s->bs, s->NB,
        s->MB, max_len, s->scale, 0, s->order.data(), s->ws, s->ws_bytes, stream);
    if (rc != PKV_OK) return rc;
  }
  // the next copy into this device buffer waits for these kernels
  if (hipEventRecord(s->consumed[s->cur], st) != hipSuccess) return PKV_ERR_HIP;
  s->in_use[s->cur] = true;
  return PKV_OK;
}

}  // extern "C"
