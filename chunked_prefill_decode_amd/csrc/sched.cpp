// Stall-free batch builder and page pool (host side of libsarathi_attn).
//
// Each iteration takes every running decode (one token each), then continues
// unfinished prefills with chunks that fill the remaining token budget, then
// admits new requests while budget and KV pages allow ("Sarathi-Serve：以
// chunked-prefills 与 stall-free batching 驯服 LLM 推理的吞吐—延迟权衡", 核心机制-2,
// Algorithm 3; "Sarathi-Serve: Chunked Prefills for Stall-Free LLM Inference",
// The mechanism).  KV lives in 16-token pages reached through per-request
// block tables ("In-flight Batching", KV Cache 管理的协同优化) and requests move
// waiting -> prefill chunks -> decode -> completed (same page, 调度状态机).
//
// Build is planned first and applied only when every check has passed, so a
// failing call leaves the state untouched.
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_set>
#include <vector>

#include "common.h"

namespace {

struct Request {
  int64_t id;
  int32_t prompt_len;   // L
  int32_t max_new;      // O
  int32_t computed;     // c: prompt tokens in the cache
  int32_t generated;    // g: output tokens produced
  std::vector<int32_t> pages;
  bool decoding() const { return computed == prompt_len; }
};

inline int32_t pages_for(int64_t tokens) { return int32_t((tokens + sa::kPageSize - 1) / sa::kPageSize); }

struct Pending {
  bool valid = false;
  int32_t num_decodes = 0;
  std::vector<int32_t> run_idx;   // index into running for each batch sequence
  std::vector<int32_t> q_len;
  std::vector<int64_t> ids;
};

}  // namespace

struct sa_sched {
  sa_sched_config cfg;
  int32_t policy = SA_POLICY_STALL_FREE;
  int32_t prefill_limit = 0;      // token cap of a baseline prefill iteration
  std::vector<Request> running;   // admission / injection order
  std::deque<Request> waiting;    // FIFO of new requests
  std::deque<int32_t> free_pages; // FIFO page pool
  std::unordered_set<int64_t> ids;
  Pending pending;
};

extern "C" {

sa_status sa_sched_create(const sa_sched_config* cfg, const int32_t* free_pages, sa_sched** out) {
  if (!cfg || !free_pages || !out) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_create: null pointer");
  if (cfg->page_size != sa::kPageSize)
    return sa::fail(SA_ERR_UNSUPPORTED, "sa_sched_create: page_size %d (only 16 is supported)", cfg->page_size);
  if (cfg->token_budget < 1 || cfg->max_blocks_per_seq < 1 || cfg->num_pages < 1)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_create: budget %d, W %d, pages %d must be >= 1",
                    cfg->token_budget, cfg->max_blocks_per_seq, cfg->num_pages);
  if (int64_t(cfg->max_blocks_per_seq) * sa::kPageSize > (int64_t(1) << 30))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_create: W too large");
  std::vector<char> seen(size_t(cfg->num_pages), 0);
  for (int32_t i = 0; i < cfg->num_pages; ++i) {
    int32_t p = free_pages[i];
    if (p < 0 || p >= cfg->num_pages || seen[size_t(p)])
      return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_create: free_pages is not a permutation (entry %d = %d)", i, p);
    seen[size_t(p)] = 1;
  }
  sa_sched* s = new (std::nothrow) sa_sched();
  if (!s) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_create: out of host memory");
  s->cfg = *cfg;
  s->free_pages.assign(free_pages, free_pages + cfg->num_pages);
  *out = s;
  return SA_OK;
}

void sa_sched_destroy(sa_sched* s) { delete s; }

sa_status sa_sched_clone(const sa_sched* src, sa_sched** out) {
  if (!src || !out) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_clone: null pointer");
  sa_sched* s = new (std::nothrow) sa_sched(*src);
  if (!s) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_clone: out of host memory");
  *out = s;
  return SA_OK;
}

sa_status sa_sched_stats(const sa_sched* s, int32_t* num_running, int32_t* num_waiting, int32_t* num_free) {
  if (!s) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_stats: null handle");
  if (num_running) *num_running = int32_t(s->running.size());
  if (num_waiting) *num_waiting = int32_t(s->waiting.size());
  if (num_free) *num_free = int32_t(s->free_pages.size());
  return SA_OK;
}

sa_status sa_sched_add_request(sa_sched* s, int64_t id, int32_t L, int32_t O, int32_t c, int32_t g) {
  if (!s) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_add_request: null handle");
  if (s->ids.count(id)) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_add_request: duplicate id %lld", (long long)id);
  const int64_t span = int64_t(s->cfg.max_blocks_per_seq) * sa::kPageSize;
  if (L < 1 || O < 1 || int64_t(L) + O - 1 > span)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_add_request: prompt %d + outputs %d - 1 must be in [1, %lld]", L, O,
                    (long long)span);
  Request r{id, L, O, c, g, {}};
  int32_t reserve = -1;
  if (c == 0 && g == 0) {
    reserve = 0;
  } else if (c > 0 && c < L && g == 0) {
    reserve = pages_for(L);               // a prefill in progress holds its whole prompt
  } else if (c == L && g >= 1 && g < O) {
    reserve = pages_for(int64_t(L) + g - 1);  // a decode holds the tokens in its cache
  } else {
    return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_add_request: inconsistent progress (computed %d of %d, generated %d of %d)",
                    c, L, g, O);
  }
  if (reserve > 0) {
    if (size_t(reserve) > s->free_pages.size())
      return sa::fail(SA_ERR_NO_PAGES, "sa_sched_add_request: needs %d pages, %zu free", reserve, s->free_pages.size());
    r.pages.assign(s->free_pages.begin(), s->free_pages.begin() + reserve);
    s->free_pages.erase(s->free_pages.begin(), s->free_pages.begin() + reserve);
    s->running.push_back(std::move(r));
  } else {
    s->waiting.push_back(std::move(r));
  }
  s->ids.insert(id);
  s->pending.valid = false;
  return SA_OK;
}

sa_status sa_sched_set_policy(sa_sched* s, int32_t policy, int32_t prefill_token_limit) {
  if (!s) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_set_policy: null handle");
  if (policy != SA_POLICY_STALL_FREE && policy != SA_POLICY_PREFILL_FIRST && policy != SA_POLICY_DECODE_FIRST)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_set_policy: unknown policy %d", policy);
  if (policy != SA_POLICY_STALL_FREE && prefill_token_limit < 1)
    return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_set_policy: prefill token limit %d", prefill_token_limit);
  s->policy = policy;
  s->prefill_limit = prefill_token_limit;
  s->pending.valid = false;
  return SA_OK;
}

sa_status sa_build_batch(sa_sched* s, sa_batch* b) {
  if (!s || !b) return sa::fail(SA_ERR_INVALID_ARG, "sa_build_batch: null pointer");
  const int32_t B = s->cfg.token_budget;
  const int32_t W = s->cfg.max_blocks_per_seq;

  // ---- plan (no mutation) ----
  struct Seq { int32_t run_idx; int32_t ctx; int32_t q; bool grow; };
  std::vector<Seq> seqs;
  seqs.reserve(s->running.size() + 8);
  int32_t n = 0, grow = 0, D = 0, admit = 0;
  size_t free_left = s->free_pages.size();
  std::vector<int32_t> admit_chunk;
  auto plan_decodes = [&](int32_t cap, const char* what) {
    for (size_t i = 0; i < s->running.size(); ++i) {
      const Request& r = s->running[i];
      if (!r.decoding()) continue;
      const int32_t pos = r.prompt_len + r.generated - 1;
      const bool g = int64_t(pos) == int64_t(sa::kPageSize) * int64_t(r.pages.size());
      grow += g;
      seqs.push_back({int32_t(i), pos, 1, g});
      ++n;
    }
    D = n;
    if (D > cap) return sa::fail(SA_ERR_BUDGET, "sa_build_batch: %d running decodes exceed the %s %d", D, what, cap);
    if (size_t(grow) > s->free_pages.size())
      return sa::fail(SA_ERR_NO_PAGES, "sa_build_batch: %d decodes need a new page, %zu free", grow, s->free_pages.size());
    free_left -= size_t(grow);
    return SA_OK;
  };
  if (s->policy == SA_POLICY_STALL_FREE) {
    sa_status st = plan_decodes(B, "budget");               // step 1: every decode
    if (st != SA_OK) return st;
    for (size_t i = 0; i < s->running.size() && n < B; ++i) {  // step 2: unfinished prefills
      const Request& r = s->running[i];
      if (r.decoding()) continue;
      const int32_t chunk = std::min(r.prompt_len - r.computed, B - n);
      seqs.push_back({int32_t(i), r.computed, chunk, false});
      n += chunk;
    }
    for (size_t w = 0; w < s->waiting.size() && n < B; ++w) {  // step 3: admissions
      const Request& r = s->waiting[w];
      const size_t need = size_t(pages_for(r.prompt_len));
      if (need > free_left) break;                             // FCFS: the head blocks
      free_left -= need;
      const int32_t chunk = std::min(r.prompt_len, B - n);
      admit_chunk.push_back(chunk);
      n += chunk;
      ++admit;
    }
  } else {
    // Baselines: an iteration is either whole prompts only (unfinished ones
    // first, then admissions) with every decode waiting, or all decodes.
    // Prefill-first admits whenever pages allow; decode-first only when
    // nothing is running.  Prompts are taken while the iteration stays within
    // the prefill token limit; the first one always.
    const int32_t cap = s->prefill_limit;
    for (size_t i = 0; i < s->running.size(); ++i) {
      const Request& r = s->running[i];
      if (r.decoding()) continue;
      const int32_t chunk = r.prompt_len - r.computed;
      if (n > 0 && n + chunk > cap) break;
      seqs.push_back({int32_t(i), r.computed, chunk, false});
      n += chunk;
    }
    const bool may_admit = s->policy == SA_POLICY_PREFILL_FIRST || s->running.empty();
    for (size_t w = 0; may_admit && w < s->waiting.size(); ++w) {
      const Request& r = s->waiting[w];
      const size_t need = size_t(pages_for(r.prompt_len));
      if (need > free_left || (n > 0 && n + r.prompt_len > cap)) break;
      free_left -= need;
      admit_chunk.push_back(r.prompt_len);
      n += r.prompt_len;
      ++admit;
    }
    if (n == 0) {
      sa_status st = plan_decodes(cap, "token limit");
      if (st != SA_OK) return st;
    }
  }
  const int32_t S = int32_t(seqs.size()) + admit;
  if (S > b->cap_seqs || n > b->cap_tokens) {
    b->num_seqs = S;
    b->num_tokens = n;
    return sa::fail(SA_ERR_CAPACITY, "sa_build_batch: needs %d sequences / %d tokens, capacity %d / %d", S, n,
                    b->cap_seqs, b->cap_tokens);
  }
  if (S > 0 && (!b->req_ids || !b->cu_seqlens_q || !b->context_lens || !b->block_tables))
    return sa::fail(SA_ERR_INVALID_ARG, "sa_build_batch: null output array");
  if (n > 0 && !b->slot_mapping) return sa::fail(SA_ERR_INVALID_ARG, "sa_build_batch: null slot_mapping");
  if (!b->cu_seqlens_q) return sa::fail(SA_ERR_INVALID_ARG, "sa_build_batch: null cu_seqlens_q");

  // ---- apply ----
  for (const Seq& q : seqs) {
    if (q.grow) {
      s->running[size_t(q.run_idx)].pages.push_back(s->free_pages.front());
      s->free_pages.pop_front();
    }
  }
  for (int32_t a = 0; a < admit; ++a) {
    Request r = std::move(s->waiting.front());
    s->waiting.pop_front();
    const int32_t need = pages_for(r.prompt_len);
    r.pages.assign(s->free_pages.begin(), s->free_pages.begin() + need);
    s->free_pages.erase(s->free_pages.begin(), s->free_pages.begin() + need);
    s->running.push_back(std::move(r));
    seqs.push_back({int32_t(s->running.size() - 1), 0, admit_chunk[size_t(a)], false});
  }

  // ---- emit ----
  Pending& p = s->pending;
  p.valid = true;
  p.num_decodes = D;
  p.run_idx.resize(size_t(S));
  p.q_len.resize(size_t(S));
  p.ids.resize(size_t(S));
  int32_t tok = 0, max_kv = 0;
  b->cu_seqlens_q[0] = 0;
  for (int32_t i = 0; i < S; ++i) {
    const Seq& q = seqs[size_t(i)];
    const Request& r = s->running[size_t(q.run_idx)];
    b->req_ids[i] = r.id;
    b->context_lens[i] = q.ctx;
    int32_t* row = b->block_tables + size_t(i) * size_t(W);
    const size_t np = r.pages.size();
    std::memcpy(row, r.pages.data(), np * sizeof(int32_t));
    std::fill(row + np, row + W, -1);
    for (int32_t t = 0; t < q.q; ++t) {
      const int32_t pos = q.ctx + t;
      b->slot_mapping[tok + t] = r.pages[size_t(pos / sa::kPageSize)] * sa::kPageSize + pos % sa::kPageSize;
    }
    tok += q.q;
    b->cu_seqlens_q[i + 1] = tok;
    max_kv = std::max(max_kv, q.ctx + q.q);
    p.run_idx[size_t(i)] = q.run_idx;
    p.q_len[size_t(i)] = q.q;
    p.ids[size_t(i)] = r.id;
  }
  b->num_seqs = S;
  b->num_decodes = D;
  b->num_prefill_chunks = S - D;
  b->num_tokens = tok;
  b->max_blocks_per_seq = W;
  b->max_kv_len = max_kv;
  return SA_OK;
}

sa_status sa_sched_commit(sa_sched* s, const sa_batch* b, int64_t* finished, int32_t cap, int32_t* num_finished) {
  if (!s || !b || !num_finished) return sa::fail(SA_ERR_INVALID_ARG, "sa_sched_commit: null pointer");
  Pending& p = s->pending;
  if (!p.valid) return sa::fail(SA_ERR_STATE, "sa_sched_commit: no pending batch (not built, or invalidated by add_request)");
  const int32_t S = int32_t(p.ids.size());
  if (b->num_seqs != S || b->num_decodes != p.num_decodes)
    return sa::fail(SA_ERR_STATE, "sa_sched_commit: batch is not the pending one (%d seqs vs %d)", b->num_seqs, S);
  for (int32_t i = 0; i < S; ++i) {
    if (b->req_ids[i] != p.ids[size_t(i)] || b->cu_seqlens_q[i + 1] - b->cu_seqlens_q[i] != p.q_len[size_t(i)])
      return sa::fail(SA_ERR_STATE, "sa_sched_commit: sequence %d differs from the pending batch", i);
  }
  // count first so that a short output array leaves the state untouched
  int32_t nfin = 0;
  for (int32_t i = 0; i < S; ++i) {
    const Request& r = s->running[size_t(p.run_idx[size_t(i)])];
    int32_t g = r.generated, c = r.computed;
    if (i < p.num_decodes) {
      ++g;
    } else {
      c += p.q_len[size_t(i)];
      if (c == r.prompt_len) g = 1;
    }
    nfin += (g == r.max_new);
  }
  if (nfin > cap || (nfin > 0 && !finished)) {
    *num_finished = nfin;
    return sa::fail(SA_ERR_CAPACITY, "sa_sched_commit: %d finished ids, capacity %d", nfin, cap);
  }
  std::vector<char> done(s->running.size(), 0);
  int32_t k = 0;
  for (int32_t i = 0; i < S; ++i) {
    Request& r = s->running[size_t(p.run_idx[size_t(i)])];
    if (i < p.num_decodes) {
      ++r.generated;
    } else {
      r.computed += p.q_len[size_t(i)];
      if (r.computed == r.prompt_len) r.generated = 1;   // the last chunk yields the first token
    }
    if (r.generated == r.max_new) {
      finished[k++] = r.id;
      done[size_t(p.run_idx[size_t(i)])] = 1;
    }
  }
  // free in batch (finish) order, each request's pages in logical order
  for (int32_t i = 0; i < k; ++i) {
    for (size_t j = 0; j < s->running.size(); ++j) {
      if (done[j] && s->running[j].id == finished[i]) {
        for (int32_t pg : s->running[j].pages) s->free_pages.push_back(pg);
        s->ids.erase(finished[i]);
        break;
      }
    }
  }
  size_t w = 0;
  for (size_t j = 0; j < s->running.size(); ++j) {
    if (!done[j]) {
      if (w != j) s->running[w] = std::move(s->running[j]);
      ++w;
    }
  }
  s->running.resize(w);
  p.valid = false;
  *num_finished = k;
  return SA_OK;
}

sa_status sa_history_slots(const sa_batch* b, int32_t* slots, int64_t cap, int64_t* count) {
  if (!b || !count) return sa::fail(SA_ERR_INVALID_ARG, "sa_history_slots: null pointer");
  int64_t total = 0;
  for (int32_t i = 0; i < b->num_seqs; ++i) total += b->context_lens[i];
  *count = total;
  if (total > cap || (total > 0 && !slots))
    return sa::fail(SA_ERR_CAPACITY, "sa_history_slots: %lld slots, capacity %lld", (long long)total, (long long)cap);
  const int32_t W = b->max_blocks_per_seq;
  int64_t k = 0;
  for (int32_t i = 0; i < b->num_seqs; ++i) {
    const int32_t* row = b->block_tables + size_t(i) * size_t(W);
    for (int32_t pos = 0; pos < b->context_lens[i]; ++pos)
      slots[k++] = row[pos / sa::kPageSize] * sa::kPageSize + pos % sa::kPageSize;
  }
  return SA_OK;
}

}  // extern "C"
