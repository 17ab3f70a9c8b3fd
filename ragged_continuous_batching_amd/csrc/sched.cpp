// Host step builder for continuous batching: the scheduling rule plus a FIFO block allocator.
//
// Hugging Face blog "Continuous batching from first principles", section "Continuous
// batching": fill m tokens per step, every decoding request first with one token, then
// prefill chunks; finished requests leave at once and waiting ones take their place.
// hassanahmed "How continuous batching speeds up LLM serving": the loop evicts finished
// requests and releases their KV blocks, admits while can_admit holds, then runs one step;
// the KV cache is kept in fixed-size blocks handed out and reclaimed on demand.
// The readings taken where the pages are silent are stated in include/cb.h.
//
// Pure host C++17: no HIP calls, so it runs and is tested without a GPU.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <string>
#include <vector>

#include "cb.h"
#include "cb_common.h"

namespace {

struct Req {
  int64_t id;
  int32_t prompt_len, out_len;
  int32_t pre_len = 0;                 // positions to prefill before decoding (prompt, or all
                                       // known tokens after a preemption)
  int32_t ctx = 0, gen = 0;
  std::vector<int32_t> blocks;
  bool done = false;
};

inline int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

}  // namespace

struct cb_sched {
  int32_t m, bs, max_num_seqs, num_blocks;
  int32_t static_b = 0;                // > 0: naive padded batches of up to this many requests
  int32_t preempt = 0, watermark = 0;  // preemption by recompute; blocks kept free at admission
  std::deque<int32_t> free_list;
  std::deque<Req> waiting;
  std::vector<Req> running;            // admission order
  // the built step awaiting commit: (index into running, rows)
  std::vector<std::pair<int32_t, int32_t>> pending;
  bool has_pending = false;
  // storage handed out through cb_step
  std::vector<int64_t> req_ids, evicted, admitted, preempted;
  std::vector<int32_t> cu, ctx, bt, slots, owner;
};

extern "C" cb_sched* cb_sched_create(int32_t token_budget, int32_t block_size, int32_t num_blocks,
                                     int32_t max_num_seqs, const int32_t* initial_free_list) {
  if (token_budget < 1 || block_size < 1 || num_blocks < 0 || max_num_seqs < 0) {
    cb::set_error("cb_sched_create: token_budget and block_size must be >= 1, counts >= 0");
    return nullptr;
  }
  cb_sched* s = new (std::nothrow) cb_sched();
  if (!s) return nullptr;
  s->m = token_budget;
  s->bs = block_size;
  s->max_num_seqs = max_num_seqs;
  s->num_blocks = num_blocks;
  if (initial_free_list) {
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_list[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        cb::set_error("cb_sched_create: initial_free_list is not a permutation of 0..num_blocks-1");
        delete s;
        return nullptr;
      }
      seen[b] = 1;
      s->free_list.push_back(b);
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) s->free_list.push_back(i);
  }
  return s;
}

extern "C" void cb_sched_destroy(cb_sched* s) { delete s; }

extern "C" cb_sched* cb_sched_clone(const cb_sched* s) {
  if (!s) return nullptr;
  cb_sched* c = new (std::nothrow) cb_sched(*s);
  if (!c) return nullptr;
  c->pending.clear();
  c->has_pending = false;
  return c;
}

extern "C" int cb_sched_set_static(cb_sched* s, int32_t batch_size) {
  if (!s || batch_size < 1) return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_set_static: batch_size must be >= 1");
  if (s->has_pending || !s->running.empty())
    return cb::fail(CB_ERR_STATE, "cb_sched_set_static: requests are already running");
  if (s->preempt) return cb::fail(CB_ERR_STATE, "cb_sched_set_static: preemption is enabled");
  s->static_b = batch_size;
  return CB_OK;
}

extern "C" int cb_sched_set_preemption(cb_sched* s, int32_t enable, int32_t watermark_blocks) {
  if (!s || watermark_blocks < 0)
    return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_set_preemption: watermark_blocks must be >= 0");
  if (s->static_b > 0 && enable) return cb::fail(CB_ERR_STATE, "cb_sched_set_preemption: not with naive batching");
  s->preempt = enable != 0;
  s->watermark = watermark_blocks;
  return CB_OK;
}

extern "C" int cb_sched_add(cb_sched* s, int64_t req_id, int32_t prompt_len, int32_t out_len) {
  if (!s || prompt_len < 1 || out_len < 1)
    return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_add: prompt_len and out_len must be >= 1");
  Req r;
  r.id = req_id;
  r.prompt_len = prompt_len;
  r.pre_len = prompt_len;
  r.out_len = out_len;
  s->waiting.push_back(std::move(r));
  return CB_OK;
}

extern "C" int cb_sched_add_cached(cb_sched* s, int64_t req_id, int32_t prompt_len, int32_t out_len,
                                   int32_t cached, int32_t generated) {
  if (!s || prompt_len < 1 || out_len < 1)
    return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_add_cached: prompt_len and out_len must be >= 1");
  bool prefill_ok = generated == 0 && cached >= 0 && cached < prompt_len;
  bool decode_ok = generated >= 1 && generated < out_len &&
                   static_cast<int64_t>(cached) == static_cast<int64_t>(prompt_len) + generated - 1;
  if (!prefill_ok && !decode_ok)
    return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_add_cached: inconsistent cached/generated state");
  if (s->has_pending) return cb::fail(CB_ERR_STATE, "cb_sched_add_cached: a built step is pending");
  int32_t need = ceil_div(cached, s->bs);
  if (need > static_cast<int32_t>(s->free_list.size()))
    return cb::fail(CB_ERR_OUT_OF_BLOCKS, "cb_sched_add_cached: free list too short");
  Req r;
  r.id = req_id;
  r.prompt_len = prompt_len;
  r.pre_len = prompt_len;
  r.out_len = out_len;
  r.ctx = cached;
  r.gen = generated;
  for (int32_t i = 0; i < need; ++i) {
    r.blocks.push_back(s->free_list.front());
    s->free_list.pop_front();
  }
  s->running.push_back(std::move(r));
  return CB_OK;
}

namespace {

// Naive batching (hassanahmed "How continuous batching speeds up LLM serving", the batch
// loop that returns results when the batch finishes; zhangchitc "continuous-batching",
// section "Naive batching: the whole batch finishes together"; Hugging Face blog, section
// "Continuous batching", batched generation with padding): up to B waiting requests start
// together, every prompt is padded to the longest one and prefilled in one step, then every
// member decodes one row per step, finished ones included, until all are done; only then do
// they leave and the next batch starts. Pad rows sit after the prompt, at positions
// prompt_len .. P-1, where causal attention keeps them out of the prompt's rows; the first
// decode row overwrites position prompt_len. The token budget m does not apply.
int build_static(cb_sched* s, std::vector<std::pair<int32_t, int32_t>>& batch, int32_t& num_decode) {
  const int32_t bs = s->bs;
  bool all_done = !s->running.empty();
  for (const auto& r : s->running) all_done = all_done && r.done;
  if (all_done) {                      // the batch has finished: everyone leaves together
    for (auto& r : s->running) {
      for (int32_t b : r.blocks) s->free_list.push_back(b);
      s->evicted.push_back(r.id);
    }
    s->running.clear();
  }
  if (s->running.empty()) {            // start the next batch with its padded prefill
    int32_t k = 0, P = 0;
    while (k < s->static_b && k < static_cast<int32_t>(s->waiting.size())) {
      const int32_t P2 = std::max(P, s->waiting[k].prompt_len);
      if (static_cast<int64_t>(k + 1) * ceil_div(P2, bs) > static_cast<int64_t>(s->free_list.size())) break;
      P = P2;
      ++k;
    }
    if (k == 0 && !s->waiting.empty())
      return cb::fail(CB_ERR_OUT_OF_BLOCKS, "cb_sched_build: free list cannot hold the padded prompt");
    for (int32_t i = 0; i < k; ++i) {
      Req r = std::move(s->waiting.front());
      s->waiting.pop_front();
      for (int32_t j = 0; j < ceil_div(P, bs); ++j) {
        r.blocks.push_back(s->free_list.front());
        s->free_list.pop_front();
      }
      s->admitted.push_back(r.id);
      s->running.push_back(std::move(r));
      batch.emplace_back(i, P);
    }
    num_decode = 0;
    return CB_OK;
  }
  int64_t need = 0;                    // one decode row for every member
  for (const auto& r : s->running)
    need += std::max<int64_t>(0, ceil_div(r.ctx + 1, bs) - static_cast<int64_t>(r.blocks.size()));
  if (need > static_cast<int64_t>(s->free_list.size()))
    return cb::fail(CB_ERR_OUT_OF_BLOCKS, "cb_sched_build: free list cannot hold the decode tokens");
  for (int32_t i = 0; i < static_cast<int32_t>(s->running.size()); ++i) {
    Req& r = s->running[i];
    while (static_cast<int32_t>(r.blocks.size()) < ceil_div(r.ctx + 1, bs)) {
      r.blocks.push_back(s->free_list.front());
      s->free_list.pop_front();
    }
    batch.emplace_back(i, 1);
  }
  num_decode = static_cast<int32_t>(batch.size());
  return CB_OK;
}

}  // namespace

extern "C" int cb_sched_build(cb_sched* s, cb_step* out) {
  if (!s || !out) return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_build: null argument");
  if (s->has_pending) return cb::fail(CB_ERR_STATE, "cb_sched_build: commit the previous step first");
  const int32_t bs = s->bs;
  s->evicted.clear();
  s->admitted.clear();
  s->preempted.clear();
  std::vector<std::pair<int32_t, int32_t>> batch;
  int32_t num_decode = 0;
  if (s->static_b > 0) {
    const int st = build_static(s, batch, num_decode);
    if (st != CB_OK) return st;
  } else {

    // 1. evict finished requests; their blocks go to the tail of the free list in table order
    {
      std::vector<Req> keep;
      keep.reserve(s->running.size());
      for (auto& r : s->running) {
        if (r.done) {
          for (int32_t b : r.blocks) s->free_list.push_back(b);
          s->evicted.push_back(r.id);
        } else {
          keep.push_back(std::move(r));
        }
      }
      s->running.swap(keep);
    }

    // 2. decode-phase requests first, one token each (at most m)
    int64_t need = 0;
    auto collect_decodes = [&]() {
      batch.clear();
      need = 0;
      for (int32_t i = 0; i < static_cast<int32_t>(s->running.size()); ++i) {
        const Req& r = s->running[i];
        if (r.ctx >= r.pre_len) {
          if (static_cast<int32_t>(batch.size()) == s->m) break;
          batch.emplace_back(i, 1);
          need += std::max<int64_t>(0, ceil_div(r.ctx + 1, bs) - static_cast<int64_t>(r.blocks.size()));
        }
      }
    };
    collect_decodes();
    // Preemption (hassanahmed, paged-memory section: when the card fills, a request is
    // evicted for a while and brought back later): the most recently admitted request gives
    // back all its blocks and returns to the head of the waiting queue; on re-admission it
    // prefills every token it has (prompt and generated), the last of which yields its next
    // token, so its output continues where it stopped.
    while (need > static_cast<int64_t>(s->free_list.size()) && s->preempt && !s->running.empty()) {
      Req r = std::move(s->running.back());
      s->running.pop_back();
      for (int32_t b : r.blocks) s->free_list.push_back(b);
      r.blocks.clear();
      r.pre_len = r.prompt_len + r.gen;
      r.ctx = 0;
      s->preempted.push_back(r.id);
      s->waiting.push_front(std::move(r));
      collect_decodes();
    }
    if (need > static_cast<int64_t>(s->free_list.size()))
      return cb::fail(CB_ERR_OUT_OF_BLOCKS, "cb_sched_build: free list cannot hold the decode tokens");
    for (auto& [i, q] : batch) {
      Req& r = s->running[i];
      while (static_cast<int32_t>(r.blocks.size()) < ceil_div(r.ctx + 1, bs)) {
        r.blocks.push_back(s->free_list.front());
        s->free_list.pop_front();
      }
    }
    num_decode = static_cast<int32_t>(batch.size());
    int64_t budget = s->m - num_decode;

    // 3. continue partly prefilled requests
    for (int32_t i = 0; i < static_cast<int32_t>(s->running.size()) && budget > 0; ++i) {
      Req& r = s->running[i];
      if (r.ctx >= r.pre_len) continue;
      int64_t cap = (static_cast<int64_t>(r.blocks.size()) + static_cast<int64_t>(s->free_list.size())) * bs - r.ctx;
      int64_t q = std::min<int64_t>({static_cast<int64_t>(r.pre_len - r.ctx), budget, cap});
      if (q <= 0) continue;
      while (static_cast<int64_t>(r.blocks.size()) < ceil_div(r.ctx + q, bs)) {
        r.blocks.push_back(s->free_list.front());
        s->free_list.pop_front();
      }
      batch.emplace_back(i, static_cast<int32_t>(q));
      budget -= q;
    }

    // 4. admit waiting requests while can_admit holds (FIFO; the first misfit stops admission)
    while (!s->waiting.empty() && budget > 0 &&
           (s->max_num_seqs == 0 || static_cast<int32_t>(s->running.size()) < s->max_num_seqs)) {
      Req& w = s->waiting.front();
      int64_t q = std::min<int64_t>(w.pre_len, budget);
      int32_t nb = ceil_div(q, bs);
      if (static_cast<int64_t>(nb) + s->watermark > static_cast<int64_t>(s->free_list.size())) break;
      Req r = std::move(w);
      s->waiting.pop_front();
      for (int32_t k = 0; k < nb; ++k) {
        r.blocks.push_back(s->free_list.front());
        s->free_list.pop_front();
      }
      s->admitted.push_back(r.id);
      s->running.push_back(std::move(r));
      batch.emplace_back(static_cast<int32_t>(s->running.size()) - 1, static_cast<int32_t>(q));
      budget -= q;
    }
  }

  // 5. emit the packed step
  const int32_t R = static_cast<int32_t>(batch.size());
  s->req_ids.assign(R, 0);
  s->cu.assign(R + 1, 0);
  s->ctx.assign(R, 0);
  int32_t maxb = 0;
  for (int32_t k = 0; k < R; ++k) {
    const Req& r = s->running[batch[k].first];
    s->req_ids[k] = r.id;
    s->ctx[k] = r.ctx;
    s->cu[k + 1] = s->cu[k] + batch[k].second;
    maxb = std::max(maxb, ceil_div(r.ctx + batch[k].second, bs));
  }
  const int32_t T = s->cu[R];
  s->bt.assign(static_cast<size_t>(R) * maxb, -1);
  s->slots.assign(T, 0);
  s->owner.assign(T, 0);
  for (int32_t k = 0; k < R; ++k) {
    const Req& r = s->running[batch[k].first];
    const int32_t q = batch[k].second;
    const int32_t nb = ceil_div(r.ctx + q, bs);
    for (int32_t j = 0; j < nb; ++j) s->bt[static_cast<size_t>(k) * maxb + j] = r.blocks[j];
    for (int32_t i = 0; i < q; ++i) {
      const int32_t p = r.ctx + i;
      s->slots[s->cu[k] + i] = r.blocks[p / bs] * bs + p % bs;
      s->owner[s->cu[k] + i] = k;
    }
  }
  s->pending = std::move(batch);
  s->has_pending = true;

  out->num_reqs = R;
  out->num_tokens = T;
  out->max_blocks_per_req = maxb;
  out->num_decode = num_decode;
  out->req_ids = s->req_ids.data();
  out->cu_q_lens = s->cu.data();
  out->ctx_lens = s->ctx.data();
  out->block_tables = s->bt.data();
  out->slot_mapping = s->slots.data();
  out->token_to_req = s->owner.data();
  out->num_evicted = static_cast<int32_t>(s->evicted.size());
  out->num_admitted = static_cast<int32_t>(s->admitted.size());
  out->evicted = s->evicted.data();
  out->admitted = s->admitted.data();
  out->num_preempted = static_cast<int32_t>(s->preempted.size());
  out->preempted = s->preempted.data();
  return CB_OK;
}

extern "C" int cb_sched_commit(cb_sched* s, const uint8_t* eos) {
  if (!s) return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_commit: null scheduler");
  if (!s->has_pending) return cb::fail(CB_ERR_STATE, "cb_sched_commit: no step to commit");
  for (size_t k = 0; k < s->pending.size(); ++k) {
    Req& r = s->running[s->pending[k].first];
    // a padded prefill row set (naive batching) ends at the prompt: pads hold no context
    r.ctx = r.ctx < r.pre_len ? std::min(r.ctx + s->pending[k].second, r.pre_len) : r.ctx + s->pending[k].second;
    if (r.ctx >= r.pre_len) {         // this step produced an output token
      r.gen += 1;
      if (r.gen >= r.out_len || (eos && eos[k])) r.done = true;
    }
  }
  s->pending.clear();
  s->has_pending = false;
  return CB_OK;
}

extern "C" int cb_sched_stats(const cb_sched* s, int32_t* num_running, int32_t* num_waiting,
                              int32_t* num_free_blocks) {
  if (!s) return cb::fail(CB_ERR_INVALID_ARG, "cb_sched_stats: null scheduler");
  if (num_running) *num_running = static_cast<int32_t>(s->running.size());
  if (num_waiting) *num_waiting = static_cast<int32_t>(s->waiting.size());
  if (num_free_blocks) *num_free_blocks = static_cast<int32_t>(s->free_list.size());
  return CB_OK;
}
