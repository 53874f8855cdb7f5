// Host batch builder for one mixed step: block pool, running and waiting queues, and the
// decode-first, first-come-first-served token-budget plan.
//
// Follows "Chunked Prefill: Ending the Great Stall" §03-§04 (decodes first at one token each,
// then every waiting prompt in order takes the largest chunk that fits the rest of the budget;
// finished prompts join the decodes), "Chunked Prefill 的 Token 预算" §04-§08 and §11 (budget
// inequality, error when decodes alone exceed the budget, per-row positions / slots / block
// table / context length, atomic commit, whole-prompt reservation) and "Splitting Prefill From
// Decode Inside a Step" ("The arithmetic of chunk boundaries": reserve before the first chunk).
// The optional caps and priority policies (per-request cap, the proposed floor, partial-prefill
// and sequence caps, prefill-first / fair share / prefill quota) follow the readings documented
// with cb_sched_config in cb.h.
//
// A build runs in two phases.  Phase 1 checks everything that can fail (budget, blocks,
// capacities) and pre-allocates host memory without touching the logical state; phase 2 commits
// and writes the plan and cannot fail.  So every error leaves the builder exactly as it was.
#include <algorithm>
#include <cstdint>
#include <new>
#include <numeric>
#include <vector>

#include "cb.h"

namespace {

struct RunningReq {
  int32_t rid;
  int32_t ctx;                   // tokens in the cache
  std::vector<int32_t> blocks;
  int32_t waited = 0;            // consecutive steps this decode did not run
};

struct WaitingReq {
  int32_t rid;
  int32_t len;                   // prompt length
  int32_t done;                  // tokens already in the cache (cached prefix + chunks run)
  std::vector<int32_t> blocks;
  bool reserved;
};

inline int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

}  // namespace

struct cb_sched {
  int32_t bs = 0;
  int32_t max_chunk = 0;
  int32_t prefill_floor = 0;
  int32_t max_partial = 0;
  int32_t max_seqs = 0;
  int32_t policy = CB_POLICY_DECODE_FIRST;
  int32_t decode_share_pct = 50;
  int32_t quota_pct = 0;
  std::vector<int32_t> free_list;  // free blocks are free_list[free_head..]
  size_t free_head = 0;
  std::vector<RunningReq> running;
  std::vector<WaitingReq> waiting;
  int32_t next_id = 0;

  size_t free_count() const { return free_list.size() - free_head; }
  int32_t pop_block() { return free_list[free_head++]; }
};

extern "C" {

const char* cb_status_string(int status) {
  switch (status) {
    case CB_OK: return "ok";
    case CB_ERR_INVALID: return "invalid argument";
    case CB_ERR_DECODE_OVER_BUDGET: return "running decodes exceed the token budget";
    case CB_ERR_OUT_OF_BLOCKS: return "KV block pool exhausted";
    case CB_ERR_CAPACITY: return "output buffer too small";
    case CB_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int cb_sched_create(const cb_sched_config* cfg, cb_sched** out) {
  if (!cfg || !out || cfg->block_size < 1 || cfg->num_blocks < 0 || cfg->max_chunk < 0)
    return CB_ERR_INVALID;
  if (cfg->prefill_floor < 0 || cfg->max_partial_prefills < 0 || cfg->max_num_seqs < 0 ||
      cfg->policy < CB_POLICY_DECODE_FIRST || cfg->policy > CB_POLICY_FAIR_SHARE ||
      cfg->decode_share_pct < 0 || cfg->decode_share_pct > 99 || cfg->prefill_quota_pct < 0 ||
      cfg->prefill_quota_pct > 100)
    return CB_ERR_INVALID;
  *out = nullptr;
  try {
    auto* s = new cb_sched();
    s->bs = cfg->block_size;
    s->max_chunk = cfg->max_chunk;
    s->prefill_floor = cfg->prefill_floor;
    s->max_partial = cfg->max_partial_prefills;
    s->max_seqs = cfg->max_num_seqs;
    s->policy = cfg->policy;
    s->decode_share_pct = cfg->decode_share_pct ? cfg->decode_share_pct : 50;
    s->quota_pct = cfg->prefill_quota_pct;
    s->free_list.resize(cfg->num_blocks);
    if (cfg->free_list) {
      std::vector<char> seen(cfg->num_blocks, 0);
      for (int32_t i = 0; i < cfg->num_blocks; ++i) {
        int32_t b = cfg->free_list[i];
        if (b < 0 || b >= cfg->num_blocks || seen[b]) {
          delete s;
          return CB_ERR_INVALID;
        }
        seen[b] = 1;
        s->free_list[i] = b;
      }
    } else {
      for (int32_t i = 0; i < cfg->num_blocks; ++i) s->free_list[i] = i;
    }
    *out = s;
    return CB_OK;
  } catch (const std::bad_alloc&) {
    return CB_ERR_CAPACITY;
  }
}

void cb_sched_destroy(cb_sched* s) { delete s; }

int cb_sched_clone(const cb_sched* s, cb_sched** out) {
  if (!s || !out) return CB_ERR_INVALID;
  try {
    *out = new cb_sched(*s);
    return CB_OK;
  } catch (const std::bad_alloc&) {
    *out = nullptr;
    return CB_ERR_CAPACITY;
  }
}

int cb_sched_add_running(cb_sched* s, int32_t context_len, int32_t* req_id) {
  if (!s || context_len < 1) return CB_ERR_INVALID;
  const int32_t need = ceil_div(context_len, s->bs);
  if (static_cast<size_t>(need) > s->free_count()) return CB_ERR_OUT_OF_BLOCKS;
  try {
    RunningReq r{s->next_id, context_len, {}};
    r.blocks.reserve(need + 1);
    s->running.reserve(s->running.size() + 1);
    for (int32_t i = 0; i < need; ++i) r.blocks.push_back(s->pop_block());
    s->running.push_back(std::move(r));
  } catch (const std::bad_alloc&) {
    return CB_ERR_CAPACITY;
  }
  if (req_id) *req_id = s->next_id;
  ++s->next_id;
  return CB_OK;
}

int cb_sched_add_prompt(cb_sched* s, int32_t prompt_len, int32_t cached_len, int32_t* req_id) {
  if (!s || prompt_len < 1 || cached_len < 0 || cached_len > prompt_len - 1) return CB_ERR_INVALID;
  const int32_t need = ceil_div(cached_len, s->bs);
  if (static_cast<size_t>(need) > s->free_count()) return CB_ERR_OUT_OF_BLOCKS;
  try {
    WaitingReq w{s->next_id, prompt_len, cached_len, {}, false};
    w.blocks.reserve(ceil_div(prompt_len, s->bs));
    s->waiting.reserve(s->waiting.size() + 1);
    for (int32_t i = 0; i < need; ++i) w.blocks.push_back(s->pop_block());
    s->waiting.push_back(std::move(w));
  } catch (const std::bad_alloc&) {
    return CB_ERR_CAPACITY;
  }
  if (req_id) *req_id = s->next_id;
  ++s->next_id;
  return CB_OK;
}

int cb_sched_get_blocks(const cb_sched* s, int32_t req_id, int32_t* out, int32_t cap, int32_t* n) {
  if (!s || !n || cap < 0) return CB_ERR_INVALID;
  const std::vector<int32_t>* bl = nullptr;
  for (const auto& r : s->running)
    if (r.rid == req_id) bl = &r.blocks;
  for (const auto& w : s->waiting)
    if (w.rid == req_id) bl = &w.blocks;
  if (!bl) return CB_ERR_INVALID;
  *n = static_cast<int32_t>(bl->size());
  if (static_cast<size_t>(cap) < bl->size()) return CB_ERR_CAPACITY;
  if (!bl->empty() && !out) return CB_ERR_INVALID;
  std::copy(bl->begin(), bl->end(), out);
  return CB_OK;
}

int cb_sched_pending_prompts(const cb_sched* s, int32_t* n) {
  if (!s || !n) return CB_ERR_INVALID;
  int32_t c = 0;
  for (const auto& w : s->waiting) c += (w.done < w.len);
  *n = c;
  return CB_OK;
}

int cb_sched_free_blocks(const cb_sched* s, int32_t* n) {
  if (!s || !n) return CB_ERR_INVALID;
  *n = static_cast<int32_t>(s->free_count());
  return CB_OK;
}

int cb_sched_finish(cb_sched* s, int32_t req_id) {
  if (!s) return CB_ERR_INVALID;
  std::vector<int32_t>* bl = nullptr;
  size_t ri = s->running.size(), wi = s->waiting.size();
  for (size_t i = 0; i < s->running.size(); ++i)
    if (s->running[i].rid == req_id) { ri = i; bl = &s->running[i].blocks; }
  for (size_t i = 0; i < s->waiting.size() && !bl; ++i)
    if (s->waiting[i].rid == req_id && s->waiting[i].done == s->waiting[i].len) { wi = i; bl = &s->waiting[i].blocks; }
  if (!bl) return CB_ERR_INVALID;
  try {
    if (s->free_head > 0 && s->free_head * 2 >= s->free_list.size()) {   // drop the used prefix
      s->free_list.erase(s->free_list.begin(), s->free_list.begin() + s->free_head);
      s->free_head = 0;
    }
    s->free_list.insert(s->free_list.end(), bl->begin(), bl->end());
  } catch (const std::bad_alloc&) {
    return CB_ERR_CAPACITY;
  }
  if (ri < s->running.size()) s->running.erase(s->running.begin() + ri);
  else s->waiting.erase(s->waiting.begin() + wi);
  return CB_OK;
}

}  // extern "C"

namespace {

int build_step_impl(cb_sched* s, int32_t token_budget, cb_step* out) {
  const int32_t bs = s->bs;

  // ---------------- phase 1: plan without touching the logical state ----------------
  // Decode candidates are the running requests in order, then prompts that finished last step
  // (FCFS); candidate i < n_run is running[i], the others graduating[i - n_run].
  std::vector<int32_t> graduating;  // indices into waiting
  for (size_t i = 0; i < s->waiting.size(); ++i)
    if (s->waiting[i].done == s->waiting[i].len) graduating.push_back(static_cast<int32_t>(i));
  const int64_t n_run = static_cast<int64_t>(s->running.size());
  const int64_t nd_all = n_run + static_cast<int64_t>(graduating.size());
  const int64_t n_prompts = static_cast<int64_t>(s->waiting.size() - graduating.size());
  auto cand_ctx = [&](int64_t i) { return i < n_run ? s->running[i].ctx : s->waiting[graduating[i - n_run]].len; };
  auto cand_nblocks = [&](int64_t i) {
    return static_cast<int64_t>(i < n_run ? s->running[i].blocks.size() : s->waiting[graduating[i - n_run]].blocks.size());
  };
  auto cand_waited = [&](int64_t i) { return i < n_run ? s->running[i].waited : 0; };
  // A decode at position ctx needs a fresh block when its blocks are exactly full.
  auto needs_block = [&](int64_t i) { return static_cast<int64_t>(cand_ctx(i)) == static_cast<int64_t>(bs) * cand_nblocks(i); };

  const int64_t seq_cap = s->max_seqs > 0 ? s->max_seqs : nd_all + n_prompts;
  const bool strict = s->policy == CB_POLICY_DECODE_FIRST && s->quota_pct == 0;
  int64_t dec_limit = 0;
  if (strict) {
    if (nd_all > token_budget || nd_all > seq_cap) return CB_ERR_DECODE_OVER_BUDGET;
    dec_limit = nd_all;
  } else if (s->policy == CB_POLICY_DECODE_FIRST) {
    const int64_t reserve = n_prompts > 0 ? (static_cast<int64_t>(s->quota_pct) * token_budget + 99) / 100 : 0;
    dec_limit = std::min({nd_all, token_budget - reserve, seq_cap});
  } else if (s->policy == CB_POLICY_FAIR_SHARE) {
    dec_limit = std::min({nd_all, (static_cast<int64_t>(s->decode_share_pct) * token_budget + 99) / 100, seq_cap});
  }
  // Longest-waiting decodes first, running order among equals.
  std::vector<int32_t> order(static_cast<size_t>(nd_all));
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return cand_waited(x) > cand_waited(y); });
  std::vector<char> chosen(static_cast<size_t>(nd_all), 0);
  for (int64_t k = 0; k < dec_limit; ++k) chosen[order[k]] = 1;
  int64_t n_chosen = dec_limit;
  int64_t left = token_budget - n_chosen;
  int64_t nseq = n_chosen;
  // Blocks of the chosen decodes come before any prompt's reservation.
  int64_t free_avail = static_cast<int64_t>(s->free_count());
  for (int64_t i = 0; i < nd_all; ++i) free_avail -= (chosen[i] && needs_block(i));
  if (free_avail < 0) return CB_ERR_OUT_OF_BLOCKS;

  // Prompt walk, first pass (FCFS).
  struct Chunk { int32_t widx; int64_t take; int32_t reserve; };
  std::vector<Chunk> chunks;
  int64_t partial = 0;
  for (size_t i = 0; i < s->waiting.size(); ++i) {
    const auto& w = s->waiting[i];
    if (w.done == w.len) continue;  // graduating this step
    if (left == 0 || nseq >= seq_cap) break;
    const int64_t rem = w.len - w.done;
    int64_t g = std::min(rem, left);
    if (s->max_chunk > 0) g = std::min<int64_t>(g, s->max_chunk);
    if (s->prefill_floor > 0) g = std::min<int64_t>(g, s->prefill_floor);
    if (s->max_partial > 0 && g < rem && partial >= s->max_partial) continue;  // skipped this step
    int32_t reserve = 0;
    if (!w.reserved) {
      reserve = ceil_div(w.len, bs) - static_cast<int32_t>(w.blocks.size());
      if (reserve > free_avail) break;  // strict FCFS: the head waits for blocks
      free_avail -= reserve;
    }
    chunks.push_back({static_cast<int32_t>(i), g, reserve});
    partial += g < rem;
    ++nseq;
    left -= g;
  }
  // Floor: the budget left is shared evenly among the admitted prompts with tokens to go.
  if (s->prefill_floor > 0) {
    auto room = [&](const Chunk& c) {
      const auto& w = s->waiting[c.widx];
      int64_t top = w.len - w.done;
      if (s->max_chunk > 0) top = std::min<int64_t>(top, s->max_chunk);
      return top - c.take;
    };
    while (left > 0) {
      int64_t n_active = 0;
      for (const auto& c : chunks) n_active += room(c) > 0;
      if (n_active == 0) break;
      const int64_t share = left / n_active;
      if (share == 0) {
        for (auto& c : chunks) {
          if (left == 0) break;
          if (room(c) > 0) {
            ++c.take;
            --left;
          }
        }
        break;
      }
      std::vector<char> active(chunks.size());
      for (size_t k = 0; k < chunks.size(); ++k) active[k] = room(chunks[k]) > 0;
      for (size_t k = 0; k < chunks.size(); ++k) {
        if (!active[k]) continue;
        const int64_t d = std::min(room(chunks[k]), share);
        chunks[k].take += d;
        left -= d;
      }
    }
  }
  // Decodes that did not get their turn take what the prompts left (every mode but plain
  // decode-first, where all of them already run).
  if (!strict && left > 0) {
    int64_t extra = std::min({nd_all - n_chosen, left, seq_cap - nseq});
    for (int64_t k = 0; k < nd_all && extra > 0; ++k) {
      const int32_t i = order[k];
      if (chosen[i]) continue;
      chosen[i] = 1;
      free_avail -= needs_block(i);
      --extra;
      ++n_chosen;
      ++nseq;
      --left;
    }
    if (free_avail < 0) return CB_ERR_OUT_OF_BLOCKS;
  }
  const int64_t nd = n_chosen;

  int64_t blocks_emitted = 0;
  int32_t max_ctx = 0, max_dctx = 0;
  for (int64_t i = 0; i < nd_all; ++i) {
    if (!chosen[i]) continue;
    blocks_emitted += ceil_div(cand_ctx(i) + 1, bs);
    max_dctx = std::max(max_dctx, cand_ctx(i) + 1);
  }
  max_ctx = max_dctx;
  int32_t max_q = nd > 0 ? 1 : 0;
  for (const auto& c : chunks) {
    const auto& w = s->waiting[c.widx];
    max_q = std::max<int32_t>(max_q, static_cast<int32_t>(c.take));
    const int32_t ctx = w.done + static_cast<int32_t>(c.take);
    blocks_emitted += ceil_div(ctx, bs);
    max_ctx = std::max(max_ctx, ctx);
  }

  const int64_t num_seqs = nd + static_cast<int64_t>(chunks.size());
  const int64_t T = token_budget - left;
  if (num_seqs > out->cap_seqs || T > out->cap_tokens || blocks_emitted > out->cap_blocks) {
    out->cap_seqs = static_cast<int32_t>(num_seqs);
    out->cap_tokens = static_cast<int32_t>(T);
    out->cap_blocks = static_cast<int32_t>(blocks_emitted);
    return CB_ERR_CAPACITY;
  }
  if (!out->seq_ids || !out->cu_seqlens_q || !out->context_lens || !out->cu_blocks ||
      (!out->block_table && blocks_emitted) || (!out->positions && T) ||
      (!out->slot_mapping && T))
    return CB_ERR_INVALID;

  // Reserve host memory up front (capacity only; the logical state is untouched) so that
  // phase 2 cannot fail.  A bad_alloc here propagates to the caller of this function.
  s->running.reserve(s->running.size() + graduating.size());
  for (auto& r : s->running) r.blocks.reserve(r.blocks.size() + 1);
  for (int32_t i : graduating) s->waiting[i].blocks.reserve(s->waiting[i].blocks.size() + 1);
  for (const auto& c : chunks) s->waiting[c.widx].blocks.reserve(ceil_div(s->waiting[c.widx].len, bs));

  // ---------------- phase 2: commit and emit (no failure past this point) ----------------
  for (int32_t i : graduating) {
    auto& w = s->waiting[i];
    s->running.push_back(RunningReq{w.rid, w.len, std::move(w.blocks), 0});
  }

  int32_t seq = 0, row = 0, nblk = 0;
  out->cu_seqlens_q[0] = 0;
  out->cu_blocks[0] = 0;
  auto emit = [&](int32_t rid, int32_t first, int32_t n, const std::vector<int32_t>& blocks) {
    const int32_t ctx = first + n;
    out->seq_ids[seq] = rid;
    out->context_lens[seq] = ctx;
    const int32_t nb = ceil_div(ctx, bs);
    for (int32_t j = 0; j < nb; ++j) out->block_table[nblk + j] = blocks[j];
    nblk += nb;
    for (int32_t p = first; p < ctx; ++p, ++row) {
      out->positions[row] = p;
      out->slot_mapping[row] = blocks[p / bs] * bs + p % bs;
    }
    ++seq;
    out->cu_seqlens_q[seq] = row;
    out->cu_blocks[seq] = nblk;
  };

  for (size_t i = 0; i < s->running.size(); ++i) {
    auto& r = s->running[i];
    if (!chosen[i]) {
      ++r.waited;
      continue;
    }
    r.waited = 0;
    if (static_cast<int64_t>(r.ctx) == static_cast<int64_t>(bs) * static_cast<int64_t>(r.blocks.size()))
      r.blocks.push_back(s->pop_block());
    emit(r.rid, r.ctx, 1, r.blocks);
    r.ctx += 1;
  }
  for (const auto& c : chunks) {
    auto& w = s->waiting[c.widx];
    if (!w.reserved) {
      for (int32_t j = 0; j < c.reserve; ++j) w.blocks.push_back(s->pop_block());
      w.reserved = true;
    }
    emit(w.rid, w.done, static_cast<int32_t>(c.take), w.blocks);
    w.done += static_cast<int32_t>(c.take);
  }
  if (!graduating.empty()) {  // compact the queue in place (no allocation)
    size_t g = 0, wpos = 0;
    for (size_t i = 0; i < s->waiting.size(); ++i) {
      if (g < graduating.size() && static_cast<size_t>(graduating[g]) == i) {
        ++g;
        continue;
      }
      if (wpos != i) s->waiting[wpos] = std::move(s->waiting[i]);
      ++wpos;
    }
    s->waiting.erase(s->waiting.begin() + wpos, s->waiting.end());
  }

  out->num_seqs = seq;
  out->num_decodes = static_cast<int32_t>(nd);
  out->num_tokens = row;
  out->num_prefill_tokens = row - static_cast<int32_t>(nd);
  out->unused_tokens = static_cast<int32_t>(left);
  out->max_q_len = max_q;
  out->max_context_len = max_ctx;
  out->max_decode_context_len = max_dctx;
  out->num_blocks_emitted = nblk;
  return CB_OK;
}

}  // namespace

extern "C" int cb_build_step(cb_sched* s, int32_t token_budget, cb_step* out) {
  if (!s || !out || token_budget < 1) return CB_ERR_INVALID;
  try {
    return build_step_impl(s, token_budget, out);
  } catch (const std::bad_alloc&) {  // only phase 1 allocates: the state is unchanged
    return CB_ERR_CAPACITY;
  }
}
