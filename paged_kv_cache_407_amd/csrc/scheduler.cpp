// Iteration-level (continuous batching) scheduler over the host block
// manager: which requests run in each forward step, and the block tables,
// sequence lengths and slot mapping the kernels need for that step.
//
// It follows the scheduler of "LLM 推理引擎 Continuous Batching 与
// PagedAttention：从 vLLM 原理到生产级部署实战":
// * §2.2: at every step boundary, finished requests release their blocks,
//   waiting requests are admitted in arrival order while the running set is
//   below max_batch_size and their prompt's blocks can be taken (the first
//   one that does not fit stays at the head of the queue and admission
//   stops); the batch takes prefill work first, within max_num_tokens, then
//   decode requests until the batch holds max_batch_size requests;
// * §4.3 (chunked prefill): a prompt that does not fit the remaining token
//   budget is prefilled in chunks over several steps, each chunk attending
//   to the prompt's already written prefix;
// * §5.4 (preemption by recompute): when the decode requests of a step need
//   more new blocks than are free, the most recently admitted running
//   request is preempted: its blocks are freed and it returns to the head of
//   the waiting queue, its generated tokens appended to its prompt, so that
//   its KV is recomputed when it is admitted again.
// A request is prefilled (its prompt's KV written), then takes one decode
// step per generated token; it finishes after max_new_tokens decode steps.
//
// Plain host code (no device calls), not thread-safe.
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <new>
#include <unordered_set>
#include <vector>

#include "pkv.h"

struct pkv_scheduler {
  struct Req {
    int64_t id;
    int32_t prompt;     // tokens to prefill (grows on preemption)
    int32_t max_new;    // decode steps still to run
    int32_t computed;   // prompt tokens whose KV is written
    int32_t generated;  // decode steps done since (re)admission
  };
  pkv_block_manager *bm;
  int32_t max_batch, max_tokens, block_size, max_seq_len;
  std::deque<Req> waiting;
  std::vector<Req> running;  // admission order
  // the previous step's plan, committed at the start of the next step
  std::vector<std::pair<int64_t, int32_t>> planned_prefill;  // (id, chunk)
  std::vector<int64_t> planned_decode;
  std::unordered_set<int64_t> known;

  Req *find_running(int64_t id) {
    for (Req &r : running)
      if (r.id == id) return &r;
    return nullptr;
  }
  static bool decoding(const Req &r) {
    return r.computed == r.prompt && r.generated < r.max_new;
  }
  // The step's batch: prefill chunks (running index, tokens) in admission
  // order within the token budget, then every decoding request while the
  // batch has rows left.
  void compose(std::vector<std::pair<size_t, int32_t>> &pf, std::vector<size_t> &dec) const {
    pf.clear();
    dec.clear();
    int32_t tokens = 0, rows = 0;
    for (size_t i = 0; i < running.size(); ++i) {
      const Req &r = running[i];
      if (r.computed == r.prompt) continue;
      if (rows >= max_batch || tokens >= max_tokens) break;
      const int32_t n = std::min(r.prompt - r.computed, max_tokens - tokens);
      pf.push_back({i, n});
      tokens += n;
      ++rows;
    }
    for (size_t i = 0; i < running.size() && rows < max_batch; ++i)
      if (decoding(running[i])) {
        dec.push_back(i);
        ++rows;
      }
  }
};


extern "C" {

pkv_scheduler *pkv_sched_create(pkv_block_manager *bm, int32_t max_batch_size,
                                int32_t max_num_tokens, int32_t max_seq_len) {
  if (!bm || max_batch_size <= 0 || max_num_tokens <= 0 || max_seq_len <= 0)
    return nullptr;
  pkv_scheduler *s = new (std::nothrow) pkv_scheduler();
  if (!s) return nullptr;
  s->bm = bm;
  s->max_batch = max_batch_size;
  s->max_tokens = max_num_tokens;
  s->max_seq_len = max_seq_len;
  s->block_size = pkv_bm_block_size(bm);
  return s;
}

void pkv_sched_destroy(pkv_scheduler *s) { delete s; }

int pkv_sched_add_request(pkv_scheduler *s, int64_t request_id, int32_t prompt_len,
                          int32_t max_new_tokens) {
  if (!s || prompt_len <= 0 || max_new_tokens < 0 ||
      (int64_t)prompt_len + max_new_tokens > s->max_seq_len || s->known.count(request_id))
    return PKV_ERR_INVALID;
  s->known.insert(request_id);
  s->waiting.push_back({request_id, prompt_len, max_new_tokens, 0, 0});
  return PKV_OK;
}

int32_t pkv_sched_num_waiting(const pkv_scheduler *s) {
  return s ? (int32_t)s->waiting.size() : -1;
}
int32_t pkv_sched_num_running(const pkv_scheduler *s) {
  return s ? (int32_t)s->running.size() : -1;
}

int pkv_sched_step(pkv_scheduler *s, int32_t max_blocks_per_seq, int32_t pad_block,
                   pkv_step_plan *plan, int64_t *prefill_ids, int32_t *cu_q_lens,
                   int32_t *prefill_tables, int32_t *prefill_lens, int64_t *decode_ids,
                   int32_t *decode_tables, int32_t *decode_lens, int32_t *slot_mapping,
                   int64_t *finished_ids, int64_t *preempted_ids) {
  if (!s || !plan || !prefill_ids || !cu_q_lens || !prefill_tables || !prefill_lens ||
      !decode_ids || !decode_tables || !decode_lens || !slot_mapping ||
      (int64_t)max_blocks_per_seq * s->block_size < s->max_seq_len)
    return PKV_ERR_INVALID;
  pkv_block_manager *bm = s->bm;
  const int32_t bs = s->block_size;
  *plan = pkv_step_plan{};

  // 0. commit the previous step: prefill chunks written, decode steps done
  for (auto &pc : s->planned_prefill)
    if (auto *r = s->find_running(pc.first)) r->computed += pc.second;
  for (int64_t id : s->planned_decode)
    if (auto *r = s->find_running(id)) ++r->generated;
  s->planned_prefill.clear();
  s->planned_decode.clear();

  // 1. finished requests release their blocks
  for (size_t i = 0; i < s->running.size();) {
    const auto &r = s->running[i];
    if (r.computed == r.prompt && r.generated == r.max_new) {
      pkv_bm_free(bm, r.id);
      s->known.erase(r.id);
      if (finished_ids) finished_ids[plan->num_finished] = r.id;
      ++plan->num_finished;
      s->running.erase(s->running.begin() + i);
    } else {
      ++i;
    }
  }

  // 2. admission in arrival order; the first request whose prompt's blocks
  //    are not free stays at the head
  while ((int32_t)s->running.size() < s->max_batch && !s->waiting.empty()) {
    if (pkv_bm_allocate(bm, s->waiting.front().id, s->waiting.front().prompt) != PKV_OK)
      break;
    s->running.push_back(s->waiting.front());
    s->waiting.pop_front();
  }

  // 3. preemption by recompute until the decode rows' new blocks are free
  std::vector<std::pair<size_t, int32_t>> pf;
  std::vector<size_t> dec;
  for (;;) {
    s->compose(pf, dec);
    int32_t need = 0;
    for (size_t i : dec)
      if (pkv_bm_seq_len(bm, s->running[i].id) % bs == 0) ++need;
    if (need <= pkv_bm_num_free(bm) || s->running.empty()) break;
    pkv_scheduler::Req v = s->running.back();
    s->running.pop_back();
    pkv_bm_free(bm, v.id);
    v.prompt += v.generated;   // the generated tokens are recomputed too
    v.max_new -= v.generated;
    v.computed = 0;
    v.generated = 0;
    s->waiting.push_front(v);
    if (preempted_ids) preempted_ids[plan->num_preempted] = v.id;
    ++plan->num_preempted;
  }

  // 4. the plan: prefill rows first (slots of the chunk's positions, seq_len
  //    = prefix + chunk), then one appended slot per decode row
  int32_t tokens = 0;
  cu_q_lens[0] = 0;
  for (auto &[i, n] : pf) {
    pkv_scheduler::Req &r = s->running[i];
    const int32_t p = plan->num_prefill++;
    prefill_ids[p] = r.id;
    int rc = pkv_bm_build_tables(bm, &r.id, 1, max_blocks_per_seq, pad_block,
                                 prefill_tables + (int64_t)p * max_blocks_per_seq,
                                 &prefill_lens[p]);
    if (rc == PKV_OK) rc = pkv_bm_slots(bm, r.id, r.computed, n, slot_mapping + tokens);
    if (rc != PKV_OK) return rc;
    prefill_lens[p] = r.computed + n;
    tokens += n;
    cu_q_lens[p + 1] = tokens;
    s->planned_prefill.push_back({r.id, n});
  }
  plan->num_prefill_tokens = tokens;
  for (size_t i : dec) {
    pkv_scheduler::Req &r = s->running[i];
    const int32_t d = plan->num_decode++;
    int rc = pkv_bm_append_token(bm, r.id, &slot_mapping[tokens]);
    if (rc == PKV_OK)
      rc = pkv_bm_build_tables(bm, &r.id, 1, max_blocks_per_seq, pad_block,
                               decode_tables + (int64_t)d * max_blocks_per_seq,
                               &decode_lens[d]);
    if (rc != PKV_OK) return rc;  // cannot happen after step 3
    decode_ids[d] = r.id;
    ++tokens;
    s->planned_decode.push_back(r.id);
  }
  plan->num_new_tokens = tokens;
  return PKV_OK;
}

}  // extern "C"
