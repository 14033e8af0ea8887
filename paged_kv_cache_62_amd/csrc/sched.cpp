// sched.cpp -- continuous-batching step scheduler of libpkv (host only).
//
// One call plans one decode step over the pool's allocator, in the order of
// "vLLM核心概念" §3.3: retire finished requests and free their blocks, admit
// from the waiting queue while free blocks allow ("无 vLLM 环境下的 Paged-KV
// 与连续批处理调度" §3.1: admission checks the free page blocks, EOS and the
// length limit end a request and its blocks come back at once), then give
// every running request its next token position. A position that needs a
// block the queue cannot give makes the request wait ("连续批处理与KV缓存"
// §4.2, append_block) and pauses admissions until blocks are freed (§4.4).
// When every running request waits, nothing would ever free a block; the
// most recently admitted request is then preempted: it gives its blocks back
// and returns to the front of the queue, to be written again in full.

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <deque>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "host.h"

namespace {

// Argument errors go to the same per-thread message as the pool's.
pkv_status sfail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  pkv::set_last_error(buf);
  return st;
}

struct Request {
  int64_t id;
  int32_t prompt_len;      // tokens written at admission (prefix included)
  int32_t max_new;         // tokens still allowed to be decoded
  int64_t prefix;          // pool sequence whose blocks start the prompt, or -1
  int32_t prefix_len = 0;  // its length at submission
  int32_t len = 0;         // tokens held while running
  int32_t generated = 0;   // tokens decoded since admission
};

}  // namespace

struct pkv_sched {
  pkv_pool* pool = nullptr;
  pkv_sched_config cfg{};
  int32_t bs = 0, nblocks = 0, max_blocks = 0;
  std::deque<Request> waiting;
  std::vector<Request> running;  // admission order
  std::unordered_set<int64_t> ids;        // queued or running
  std::unordered_set<int64_t> last_batch; // the previous step's batch
  bool paused = false;
  pkv_sched_stats st{};
  // plan storage
  std::vector<int64_t> seqs, slots, prefill_seqs, prefill_slots;
  std::vector<int32_t> tables, lens, prefill_first, prefill_tokens;
  std::vector<pkv_event> events;
};

namespace {

int64_t free_blocks(const pkv_sched* s) { return pkv::pool_free_blocks(s->pool); }

// New blocks the prompt of r takes at admission: its logical blocks minus
// the full blocks of a shared prefix (a partly filled prefix block is copied
// on the first write into it, so it counts as new).
int64_t admission_blocks(const pkv_sched* s, const Request& r) {
  const int64_t bs = s->bs;
  const int64_t total = (r.prompt_len + bs - 1) / bs;
  if (r.prefix < 0) return total;
  if (r.prompt_len == r.prefix_len) return 0;  // the first decode token copies the partial block
  return total - r.prefix_len / bs;
}

void event(pkv_sched* s, int64_t id, int32_t kind) { s->events.push_back(pkv_event{id, kind, 0}); }

}  // namespace

extern "C" {

pkv_status pkv_sched_create(pkv_pool* pool, const pkv_sched_config* cfg, pkv_sched** out) {
  if (!out) return sfail(PKV_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!pool || !cfg) return sfail(PKV_ERR_INVALID_ARG, "NULL pool or config");
  if (cfg->max_batch < 1 || cfg->max_model_len < 2 || cfg->reserve_blocks < 0)
    return sfail(PKV_ERR_INVALID_ARG, "max_batch %d >= 1, max_model_len %d >= 2, reserve_blocks %d >= 0",
                 cfg->max_batch, cfg->max_model_len, cfg->reserve_blocks);
  if (cfg->batch_order != PKV_BATCH_ADMISSION && cfg->batch_order != PKV_BATCH_LONGEST_FIRST)
    return sfail(PKV_ERR_INVALID_ARG, "batch_order %d", cfg->batch_order);
  pkv_stats ps{};
  pkv_status e = pkv_pool_stats(pool, &ps);
  if (e != PKV_OK) return e;
  auto* s = new pkv_sched;
  s->pool = pool;
  s->cfg = *cfg;
  s->bs = pkv::pool_block_size(pool);
  s->nblocks = (int32_t)ps.total_blocks;
  s->max_blocks = (cfg->max_model_len + s->bs - 1) / s->bs;
  s->st.total_blocks = ps.total_blocks;
  *out = s;
  return PKV_OK;
}

void pkv_sched_destroy(pkv_sched* s) {
  if (!s) return;
  for (const Request& r : s->running) pkv_seq_free(s->pool, r.id);
  delete s;
}

pkv_status pkv_sched_submit(pkv_sched* s, int64_t request, int32_t prompt_len, int32_t max_new_tokens,
                            int64_t prefix_seq) {
  if (!s) return sfail(PKV_ERR_INVALID_ARG, "scheduler is NULL");
  if (prompt_len < 1 || max_new_tokens < 1)
    return sfail(PKV_ERR_INVALID_ARG, "prompt_len %d and max_new_tokens %d must be >= 1", prompt_len,
                 max_new_tokens);
  if (prompt_len >= s->cfg.max_model_len)
    return sfail(PKV_ERR_INVALID_ARG, "prompt_len %d leaves no room below max_model_len %d", prompt_len,
                 s->cfg.max_model_len);
  const int64_t most = std::min<int64_t>((int64_t)prompt_len + max_new_tokens, s->cfg.max_model_len);
  if ((most + s->bs - 1) / s->bs > s->nblocks)
    return sfail(PKV_ERR_INVALID_ARG, "a request of up to %lld tokens needs more blocks than the pool has (%d)",
                 (long long)most, s->nblocks);
  int64_t dummy = 0;
  if (s->ids.count(request) || pkv_seq_length(s->pool, request, &dummy) == PKV_OK)
    return sfail(PKV_ERR_SEQ_EXISTS, "request id %lld is in use", (long long)request);
  Request r{request, prompt_len, max_new_tokens, prefix_seq < 0 ? -1 : prefix_seq};
  if (r.prefix >= 0) {
    int64_t plen = 0;
    if (pkv_seq_length(s->pool, r.prefix, &plen) != PKV_OK)
      return sfail(PKV_ERR_UNKNOWN_SEQ, "prefix sequence %lld is not in the pool", (long long)r.prefix);
    if (plen > prompt_len)
      return sfail(PKV_ERR_INVALID_ARG, "prefix of %lld tokens is longer than the prompt (%d)", (long long)plen,
                   prompt_len);
    r.prefix_len = (int32_t)plen;
  }
  s->waiting.push_back(r);
  s->ids.insert(request);
  return PKV_OK;
}

pkv_status pkv_sched_step(pkv_sched* s, const int64_t* eos, int32_t n_eos, pkv_step_plan* plan, void* stream) {
  if (!s || !plan) return sfail(PKV_ERR_INVALID_ARG, "NULL scheduler or plan");
  if (n_eos < 0 || (n_eos > 0 && !eos)) return sfail(PKV_ERR_INVALID_ARG, "bad eos list");
  std::unordered_set<int64_t> eos_set;
  for (int32_t i = 0; i < n_eos; ++i) {
    if (!s->last_batch.count(eos[i]))
      return sfail(PKV_ERR_INVALID_ARG, "eos request %lld was not in the previous batch", (long long)eos[i]);
    eos_set.insert(eos[i]);
  }
  s->events.clear();
  s->prefill_seqs.clear();
  s->prefill_first.clear();
  s->prefill_tokens.clear();
  s->prefill_slots.clear();

  // 1. retire
  {
    std::vector<Request> keep;
    keep.reserve(s->running.size());
    bool freed = false;
    for (const Request& r : s->running) {
      int32_t kind = 0;
      if (eos_set.count(r.id)) kind = PKV_EV_EOS;
      else if (r.generated >= r.max_new || r.len >= s->cfg.max_model_len) kind = PKV_EV_MAX_LENGTH;
      if (kind == 0) {
        keep.push_back(r);
        continue;
      }
      pkv_seq_free(s->pool, r.id);
      s->ids.erase(r.id);
      event(s, r.id, kind);
      (kind == PKV_EV_EOS ? s->st.finished_eos : s->st.finished_max_length) += 1;
      freed = true;
    }
    s->running.swap(keep);
    if (freed) s->paused = false;
  }

  // 2. admit
  while (!s->paused && !s->waiting.empty() && (int32_t)s->running.size() < s->cfg.max_batch) {
    Request r = s->waiting.front();
    if (admission_blocks(s, r) + s->cfg.reserve_blocks > free_blocks(s)) break;
    const size_t at = s->prefill_slots.size();
    const int32_t first = r.prefix >= 0 ? r.prefix_len : 0;
    const int32_t n = r.prompt_len - first;
    s->prefill_slots.resize(at + n);
    pkv_status e;
    if (r.prefix >= 0) {
      e = pkv_seq_fork(s->pool, r.prefix, r.id);
      if (e == PKV_OK && n > 0) {
        e = pkv_seq_append_slots(s->pool, &r.id, 1, &n, s->prefill_slots.data() + at, stream);
        if (e != PKV_OK) pkv_seq_free(s->pool, r.id);
      }
    } else {
      e = pkv_seq_allocate(s->pool, r.id, n, s->prefill_slots.data() + at);
    }
    if (e != PKV_OK) {  // cannot happen after the block count above; leave the request queued
      s->prefill_slots.resize(at);
      return e;
    }
    s->waiting.pop_front();
    r.len = r.prompt_len;
    r.generated = 0;
    s->running.push_back(r);
    s->prefill_seqs.push_back(r.id);
    s->prefill_first.push_back(first);
    s->prefill_tokens.push_back(n);
    event(s, r.id, PKV_EV_ADMIT);
    s->st.admitted += 1;
  }

  // 3. decode positions
  s->seqs.clear();
  s->slots.clear();
  std::vector<int64_t> waiting_ids;
  for (;;) {
    s->seqs.clear();
    s->slots.clear();
    waiting_ids.clear();
    for (Request& r : s->running) {
      const int32_t one = 1;
      int64_t slot = -1;
      const pkv_status e = pkv_seq_append_slots(s->pool, &r.id, 1, &one, &slot, stream);
      if (e == PKV_OK) {
        s->seqs.push_back(r.id);
        s->slots.push_back(slot);
      } else if (e == PKV_ERR_NO_FREE_BLOCK) {
        waiting_ids.push_back(r.id);
      } else {
        return e;
      }
    }
    if (!s->seqs.empty() || s->running.empty()) break;
    // every running request waits: preempt the most recently admitted one
    Request r = s->running.back();
    s->running.pop_back();
    pkv_seq_free(s->pool, r.id);
    event(s, r.id, PKV_EV_PREEMPT);
    s->st.preempted += 1;
    r.max_new -= r.generated;
    r.prompt_len = r.len;
    r.generated = 0;
    r.len = 0;
    s->waiting.push_front(r);
  }
  for (int64_t id : waiting_ids) event(s, id, PKV_EV_WAIT);
  if (!waiting_ids.empty()) s->paused = true;

  // batch: lengths, tables, decoded-token counts
  const int32_t nb = (int32_t)s->seqs.size();
  s->tables.assign((size_t)nb * s->max_blocks, -1);
  s->lens.assign(nb, 0);
  if (nb > 0) {
    const pkv_status e =
        pkv_seq_block_table(s->pool, s->seqs.data(), nb, s->max_blocks, s->tables.data(), s->lens.data());
    if (e != PKV_OK) return e;
  }
  if (s->cfg.batch_order == PKV_BATCH_LONGEST_FIRST && nb > 1) {
    // the rows permuted, longest context first (stable): decisions and
    // allocations above are those of admission order
    std::vector<int32_t> perm(nb);
    for (int32_t i = 0; i < nb; ++i) perm[i] = i;
    std::stable_sort(perm.begin(), perm.end(), [&](int32_t x, int32_t y) { return s->lens[x] > s->lens[y]; });
    std::vector<int64_t> seqs(nb), slots(nb);
    std::vector<int32_t> tables((size_t)nb * s->max_blocks), lens(nb);
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t j = perm[i];
      seqs[i] = s->seqs[j];
      slots[i] = s->slots[j];
      lens[i] = s->lens[j];
      std::copy(s->tables.begin() + (size_t)j * s->max_blocks, s->tables.begin() + (size_t)(j + 1) * s->max_blocks,
                tables.begin() + (size_t)i * s->max_blocks);
    }
    s->seqs.swap(seqs);
    s->slots.swap(slots);
    s->tables.swap(tables);
    s->lens.swap(lens);
  }
  std::unordered_set<int64_t> in_batch(s->seqs.begin(), s->seqs.end());
  for (Request& r : s->running) {
    if (!in_batch.count(r.id)) continue;
    r.len += 1;
    r.generated += 1;
    s->st.generated += 1;
  }
  s->last_batch.swap(in_batch);

  plan->num_seqs = nb;
  plan->max_blocks = s->max_blocks;
  plan->max_context_len = 0;
  for (int32_t i = 0; i < nb; ++i) plan->max_context_len = std::max(plan->max_context_len, s->lens[i]);
  plan->num_prefill = (int32_t)s->prefill_seqs.size();
  plan->prefill_total = (int32_t)s->prefill_slots.size();
  plan->num_events = (int32_t)s->events.size();
  plan->seqs = s->seqs.data();
  plan->slots = s->slots.data();
  plan->block_tables = s->tables.data();
  plan->context_lens = s->lens.data();
  plan->prefill_seqs = s->prefill_seqs.data();
  plan->prefill_first = s->prefill_first.data();
  plan->prefill_tokens = s->prefill_tokens.data();
  plan->prefill_slots = s->prefill_slots.data();
  plan->events = s->events.data();
  return PKV_OK;
}

pkv_status pkv_sched_get_stats(const pkv_sched* s, pkv_sched_stats* out) {
  if (!s || !out) return sfail(PKV_ERR_INVALID_ARG, "NULL argument");
  *out = s->st;
  out->waiting = (int64_t)s->waiting.size();
  out->running = (int64_t)s->running.size();
  pkv_stats ps{};
  pkv_pool_stats(s->pool, &ps);
  out->used_blocks = ps.used_blocks;
  out->total_blocks = ps.total_blocks;
  out->paused = s->paused ? 1 : 0;
  return PKV_OK;
}

}  // extern "C"
