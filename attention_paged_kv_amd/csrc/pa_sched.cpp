// pa_sched.cpp -- the host step planner declared in include/pa_sched.h: block pool, decode-first
// token-budget scheduler (P4 "一步的 token 预算"), exact-prefix block cache with LRU eviction by
// block (P3 §4.3) and recompute preemption.  Plain C++; no device code.
#include "pa_sched.h"

#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <memory>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_error.h"

namespace {

constexpr int kBlk = PA_BLOCK_SIZE;

// A cache key: the parent entry (block id, registration count; -1/0 for the first block) and the
// block's 16 token ids.  Exact: equality compares every field.
struct Key {
  int32_t parent = -1;
  uint32_t parent_epoch = 0;
  std::array<int32_t, kBlk> toks{};
  bool operator==(const Key& o) const {
    return parent == o.parent && parent_epoch == o.parent_epoch && toks == o.toks;
  }
};

struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)(uint32_t)k.parent ^ ((uint64_t)k.parent_epoch << 32);
    for (int32_t t : k.toks) {
      h ^= (uint64_t)(uint32_t)t + 0x9E3779B97F4A7C15ull + (h << 6) + (h >> 2);
    }
    return (size_t)h;
  }
};

enum class State { Waiting, Running };

struct Entry {
  int32_t block;
  uint32_t epoch;
};

struct Req {
  int64_t id = 0;
  std::vector<int32_t> tokens;
  int32_t prompt_len = 0;
  int32_t max_new = 0;
  int32_t generated = 0;
  int32_t computed = 0;
  std::vector<int32_t> blocks;
  std::vector<Entry> chain;     // cache entry standing for the prefix through block j
  int64_t admit_seq = -1;
  State state = State::Waiting;
  bool decoding() const {
    return computed >= prompt_len && (int64_t)tokens.size() - computed == 1;
  }
};

struct Planned {
  Req* r;
  int32_t start;
  int32_t n;
};

}  // namespace

struct pa_sched {
  pa_sched_config cfg{};
  // pool
  std::deque<int32_t> free_list;
  std::list<int32_t> lru;                           // evictable cached blocks, oldest release first
  std::vector<std::list<int32_t>::iterator> lru_pos;
  std::vector<int32_t> ref;
  std::vector<uint32_t> epoch;
  std::vector<char> cached;                         // block registered under key_of[block]
  std::vector<Key> key_of;
  std::unordered_map<Key, int32_t, KeyHash> cache;
  // requests
  std::unordered_map<int64_t, std::unique_ptr<Req>> by_id;
  std::deque<Req*> waiting;
  std::vector<Req*> running;                        // admission order
  int64_t admit_counter = 0;
  std::vector<Planned> pending;
  bool has_pending = false;
  std::vector<int64_t> preempted;
  int64_t hit_tokens = 0;

  // ---- pool ----
  int64_t avail() const { return (int64_t)free_list.size() + (int64_t)lru.size(); }

  int32_t alloc() {
    if (!free_list.empty()) {
      const int32_t b = free_list.front();
      free_list.pop_front();
      return b;
    }
    if (!lru.empty()) {
      const int32_t b = lru.front();
      lru.pop_front();
      cache.erase(key_of[b]);
      cached[b] = 0;
      return b;
    }
    return -1;
  }

  void release_block(int32_t b) {
    if (--ref[b] == 0) {
      if (cached[b]) lru_pos[b] = lru.insert(lru.end(), b);
      else free_list.push_back(b);
    }
  }

  void release(Req* r) {
    for (auto it = r->blocks.rbegin(); it != r->blocks.rend(); ++it) release_block(*it);
    r->blocks.clear();
    r->chain.clear();
  }

  void take(int32_t b) {
    if (ref[b] == 0) lru.erase(lru_pos[b]);
    ++ref[b];
  }

  int64_t blocks_needed(const Req* r, int64_t n) const {
    return (r->computed + n + kBlk - 1) / kBlk - (int64_t)r->blocks.size();
  }

  void grow(Req* r, int64_t n) {
    for (int64_t i = blocks_needed(r, n); i > 0; --i) {
      const int32_t b = alloc();   // callers checked avail() first
      ++ref[b];
      r->blocks.push_back(b);
    }
  }

  // largest m <= n whose new blocks the pool can back
  int64_t fit(const Req* r, int64_t n) const {
    const int64_t a = avail();
    if (n > 0 && blocks_needed(r, n) > a) n = ((int64_t)r->blocks.size() + a) * kBlk - r->computed;
    return std::max<int64_t>(n, 0);
  }

  Key key_for(const Req* r, int64_t j, Entry parent) const {
    Key k;
    k.parent = parent.block;
    k.parent_epoch = parent.epoch;
    std::memcpy(k.toks.data(), r->tokens.data() + j * kBlk, sizeof(int32_t) * kBlk);
    return k;
  }

  void match(Req* r) {
    if (!cfg.prefix_cache) return;
    Entry parent{-1, 0};
    const int64_t limit = ((int64_t)r->tokens.size() - 1) / kBlk;
    for (int64_t j = 0; j < limit; ++j) {
      auto it = cache.find(key_for(r, j, parent));
      if (it == cache.end()) break;
      const int32_t b = it->second;
      take(b);
      r->blocks.push_back(b);
      parent = Entry{b, epoch[b]};
      r->chain.push_back(parent);
    }
    r->computed = (int32_t)r->blocks.size() * kBlk;
    hit_tokens += r->computed;
  }

  void remove_running(Req* r) { running.erase(std::find(running.begin(), running.end(), r)); }

  void preempt(Req* r) {
    remove_running(r);
    release(r);
    r->computed = 0;
    r->state = State::Waiting;
    waiting.push_front(r);
    preempted.push_back(r->id);
  }

  void admit(Req* r) {
    r->admit_seq = admit_counter++;
    r->state = State::Running;
    running.push_back(r);
  }

  void plan_step() {
    int64_t budget = cfg.token_budget;
    const int64_t cap = cfg.max_seqs > 0 ? cfg.max_seqs : INT64_MAX;
    pending.clear();
    preempted.clear();
    std::unordered_map<int64_t, char> in_step;
    // (1) decodes, in admission order
    const std::vector<Req*> snap = running;
    for (Req* r : snap) {
      if (r->state != State::Running || !r->decoding()) continue;
      if (budget == 0 || (int64_t)pending.size() == cap) break;
      while (blocks_needed(r, 1) > 0 && avail() < 1) {
        Req* victim = nullptr;
        for (auto it = running.rbegin(); it != running.rend(); ++it)
          if (!in_step.count((*it)->id)) { victim = *it; break; }   // newest admission first
        preempt(victim);
        if (victim == r) break;
      }
      if (r->state != State::Running) continue;
      grow(r, 1);
      pending.push_back(Planned{r, r->computed, 1});
      in_step[r->id] = 1;
      budget -= 1;
    }
    // (2) prefills: running ones, then the waiting queue
    const std::vector<Req*> snap2 = running;
    for (Req* r : snap2) {
      if (r->decoding() || in_step.count(r->id)) continue;
      if (budget == 0 || (int64_t)pending.size() == cap) break;
      const int64_t n = fit(r, std::min<int64_t>((int64_t)r->tokens.size() - r->computed, budget));
      if (n == 0) break;
      grow(r, n);
      pending.push_back(Planned{r, r->computed, (int32_t)n});
      in_step[r->id] = 1;
      budget -= n;
    }
    while (!waiting.empty() && budget > 0 && (int64_t)pending.size() < cap && preempted.empty()) {
      Req* r = waiting.front();
      match(r);
      const int64_t n = fit(r, std::min<int64_t>((int64_t)r->tokens.size() - r->computed, budget));
      if (n == 0) {
        hit_tokens -= r->computed;
        release(r);
        r->computed = 0;
        break;
      }
      waiting.pop_front();
      admit(r);
      grow(r, n);
      pending.push_back(Planned{r, r->computed, (int32_t)n});
      in_step[r->id] = 1;
      budget -= n;
    }
  }

  void commit_step(const int32_t* next_tokens, const int32_t* stop) {
    for (size_t i = 0; i < pending.size(); ++i) {
      Req* r = pending[i].r;
      const int32_t start = pending[i].start, n = pending[i].n;
      r->computed = start + n;
      for (int64_t j = (int64_t)r->chain.size(); j < r->computed / kBlk; ++j) {
        const int32_t b = r->blocks[j];
        if (!cfg.prefix_cache) {
          r->chain.push_back(Entry{b, epoch[b]});
          continue;
        }
        const Entry parent = j > 0 ? r->chain[j - 1] : Entry{-1, 0};
        Key k = key_for(r, j, parent);
        auto it = cache.find(k);
        if (it != cache.end()) {
          r->chain.push_back(Entry{it->second, epoch[it->second]});
        } else {
          ++epoch[b];
          cache.emplace(k, b);
          key_of[b] = k;
          cached[b] = 1;
          r->chain.push_back(Entry{b, epoch[b]});
        }
      }
      if ((int64_t)start + n == (int64_t)r->tokens.size()) {
        r->tokens.push_back(next_tokens[i]);
        r->generated += 1;
        if (r->generated >= r->max_new || (stop && stop[i])) {
          remove_running(r);
          release(r);
          by_id.erase(r->id);     // frees r
        }
      }
    }
    pending.clear();
  }
};

extern "C" {

int pa_sched_create(const pa_sched_config* cfg, pa_sched** out) {
  pa::clear_error();
  if (!out) return pa::set_error(PA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg) return pa::set_error(PA_ERR_INVALID_ARG, "config is NULL");
  if (cfg->num_blocks < 1 || cfg->max_blocks_per_seq < 1 || cfg->token_budget < 1 || cfg->max_seqs < 0 ||
      (cfg->prefix_cache != 0 && cfg->prefix_cache != 1))
    return pa::set_error(PA_ERR_INVALID_ARG, "bad planner config (num_blocks %d, max_blocks_per_seq %d, budget %d, "
                         "max_seqs %d, prefix_cache %d)", cfg->num_blocks, cfg->max_blocks_per_seq, cfg->token_budget,
                         cfg->max_seqs, cfg->prefix_cache);
  if ((int64_t)cfg->max_blocks_per_seq * kBlk > (1 << 30))
    return pa::set_error(PA_ERR_INVALID_ARG, "max_blocks_per_seq too large");
  pa_sched* s = new (std::nothrow) pa_sched();
  if (!s) return pa::set_error(PA_ERR_INVALID_ARG, "out of host memory");
  s->cfg = *cfg;
  const size_t nb = (size_t)cfg->num_blocks;
  for (int32_t b = 0; b < cfg->num_blocks; ++b) s->free_list.push_back(b);
  s->lru_pos.resize(nb);
  s->ref.assign(nb, 0);
  s->epoch.assign(nb, 0);
  s->cached.assign(nb, 0);
  s->key_of.resize(nb);
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int pa_sched_add(pa_sched* s, int64_t request_id, const int32_t* prompt, int32_t prompt_len,
                 int32_t max_new_tokens) {
  pa::clear_error();
  if (!s || (!prompt && prompt_len > 0)) return pa::set_error(PA_ERR_INVALID_ARG, "null argument");
  if (prompt_len < 1 || max_new_tokens < 1)
    return pa::set_error(PA_ERR_INVALID_ARG, "prompt_len (%d) and max_new_tokens (%d) must be >= 1", prompt_len,
                         max_new_tokens);
  if ((int64_t)prompt_len + max_new_tokens > (int64_t)s->cfg.max_blocks_per_seq * kBlk)
    return pa::set_error(PA_ERR_INVALID_ARG, "prompt_len + max_new_tokens exceeds %d tokens per request",
                         s->cfg.max_blocks_per_seq * kBlk);
  if (s->by_id.count(request_id)) return pa::set_error(PA_ERR_INVALID_ARG, "request %lld is already live", (long long)request_id);
  auto r = std::make_unique<Req>();
  r->id = request_id;
  r->tokens.assign(prompt, prompt + prompt_len);
  r->prompt_len = prompt_len;
  r->max_new = max_new_tokens;
  s->waiting.push_back(r.get());
  s->by_id.emplace(request_id, std::move(r));
  return PA_OK;
}

int pa_sched_abort(pa_sched* s, int64_t request_id) {
  pa::clear_error();
  if (!s) return pa::set_error(PA_ERR_INVALID_ARG, "null planner");
  if (s->has_pending) return pa::set_error(PA_ERR_INVALID_ARG, "commit the planned step first");
  auto it = s->by_id.find(request_id);
  if (it == s->by_id.end()) return pa::set_error(PA_ERR_INVALID_ARG, "request %lld is not live", (long long)request_id);
  Req* r = it->second.get();
  if (r->state == State::Running) s->remove_running(r);
  else s->waiting.erase(std::find(s->waiting.begin(), s->waiting.end(), r));
  s->release(r);
  s->by_id.erase(it);
  return PA_OK;
}

int pa_sched_schedule(pa_sched* s, pa_sched_batch* out) {
  pa::clear_error();
  if (!s || !out) return pa::set_error(PA_ERR_INVALID_ARG, "null argument");
  if (s->has_pending) return pa::set_error(PA_ERR_INVALID_ARG, "commit the planned step first");
  const int64_t need_seqs = s->cfg.max_seqs > 0 ? s->cfg.max_seqs : (int64_t)s->by_id.size();
  if (out->cap_tokens < s->cfg.token_budget || out->cap_seqs < need_seqs)
    return pa::set_error(PA_ERR_INVALID_ARG, "batch capacity (%d seqs, %d tokens) below %lld seqs / %d tokens",
                         out->cap_seqs, out->cap_tokens, (long long)need_seqs, s->cfg.token_budget);
  if (!out->request_ids || !out->query_start_loc || !out->seq_lens || !out->block_tables || !out->slot_mapping ||
      !out->token_ids || !out->positions || !out->samples)
    return pa::set_error(PA_ERR_INVALID_ARG, "null batch array");
  s->plan_step();
  s->has_pending = true;
  const int32_t mb = s->cfg.max_blocks_per_seq;
  int32_t t = 0;
  out->query_start_loc[0] = 0;
  for (size_t i = 0; i < s->pending.size(); ++i) {
    const Planned& p = s->pending[i];
    const Req* r = p.r;
    out->request_ids[i] = r->id;
    out->seq_lens[i] = p.start + p.n;
    int32_t* row = out->block_tables + (int64_t)i * mb;
    const size_t nbk = r->blocks.size();
    std::memcpy(row, r->blocks.data(), nbk * sizeof(int32_t));
    std::fill(row + nbk, row + mb, -1);
    for (int32_t q = p.start; q < p.start + p.n; ++q, ++t) {
      out->slot_mapping[t] = r->blocks[q / kBlk] * kBlk + q % kBlk;
      out->token_ids[t] = r->tokens[q];
      out->positions[t] = q;
    }
    out->query_start_loc[i + 1] = t;
    out->samples[i] = (int64_t)p.start + p.n == (int64_t)r->tokens.size() ? 1 : 0;
  }
  out->num_seqs = (int32_t)s->pending.size();
  out->num_tokens = t;
  return PA_OK;
}

int pa_sched_commit(pa_sched* s, const int32_t* next_tokens, const int32_t* stop) {
  pa::clear_error();
  if (!s) return pa::set_error(PA_ERR_INVALID_ARG, "null planner");
  if (!s->has_pending) return pa::set_error(PA_ERR_INVALID_ARG, "no planned step to commit");
  if (!next_tokens && !s->pending.empty()) return pa::set_error(PA_ERR_INVALID_ARG, "next_tokens is NULL");
  s->commit_step(next_tokens, stop);
  s->has_pending = false;
  return PA_OK;
}

int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* st) {
  pa::clear_error();
  if (!s || !st) return pa::set_error(PA_ERR_INVALID_ARG, "null argument");
  st->free_blocks = (int32_t)s->free_list.size();
  st->cached_blocks = (int32_t)s->cache.size();
  st->evictable_blocks = (int32_t)s->lru.size();
  st->running = (int32_t)s->running.size();
  st->waiting = (int32_t)s->waiting.size();
  st->preempted_last_step = (int32_t)s->preempted.size();
  st->hit_tokens = s->hit_tokens;
  return PA_OK;
}

int pa_sched_preempted(const pa_sched* s, int64_t* ids, int32_t cap, int32_t* n) {
  pa::clear_error();
  if (!s || !n || (cap > 0 && !ids)) return pa::set_error(PA_ERR_INVALID_ARG, "null argument");
  const int32_t m = (int32_t)s->preempted.size();
  for (int32_t i = 0; i < m && i < cap; ++i) ids[i] = s->preempted[i];
  *n = m;
  return PA_OK;
}

}  // extern "C"
