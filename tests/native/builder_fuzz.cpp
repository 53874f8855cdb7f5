// Random exercise of the host batch builder through its C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_builder_sanitizers.py: random pool geometries, free
// lists, caps and policies, running requests and prompts, steps under random budgets and array
// capacities (every error path), finishes, clones and queries.  Checks the invariants a caller
// relies on (capacities respected, prefix sums, slots inside the pool); the sanitizers check
// memory and arithmetic.  Prints one "ok:" line and returns 0 on success.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
#include "cb.h"
int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 2000;
  std::mt19937 rng(12345);
  auto U = [&](int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); };
  long steps = 0, errs[8] = {0};
  for (int it = 0; it < iters; ++it) {
    cb_sched_config cfg{};
    cfg.block_size = 1 << U(0, 6);
    cfg.num_blocks = U(0, 400);
    std::vector<int32_t> fl(cfg.num_blocks);
    for (int i = 0; i < cfg.num_blocks; ++i) fl[i] = i;
    std::shuffle(fl.begin(), fl.end(), rng);
    cfg.free_list = U(0, 1) ? fl.data() : nullptr;
    cfg.max_chunk = U(0, 3) ? 0 : U(1, 300);
    cfg.prefill_floor = U(0, 3) ? 0 : U(1, 100);
    cfg.max_partial_prefills = U(0, 3) ? 0 : U(1, 4);
    cfg.max_num_seqs = U(0, 3) ? 0 : U(1, 40);
    cfg.policy = U(0, 2);
    cfg.decode_share_pct = U(0, 3) ? 0 : U(1, 99);
    cfg.prefill_quota_pct = U(0, 3) ? 0 : U(0, 100);
    cb_sched* s = nullptr;
    if (cb_sched_create(&cfg, &s) != CB_OK) { errs[0]++; continue; }
    std::vector<int32_t> ids;
    const int nrun = U(0, 30), npr = U(0, 6);
    for (int i = 0; i < nrun; ++i) { int32_t id; if (cb_sched_add_running(s, U(1, 900), &id) == CB_OK) ids.push_back(id); else errs[1]++; }
    for (int i = 0; i < npr; ++i) { int L = U(1, 2000); int32_t id; if (cb_sched_add_prompt(s, L, U(0, L - 1), &id) == CB_OK) ids.push_back(id); else errs[2]++; }
    const int cap_seqs = U(1, 64), cap_tokens = U(1, 1024), cap_blocks = U(1, 5000);
    std::vector<int32_t> seq_ids(cap_seqs), cu_q(cap_seqs + 1), ctx(cap_seqs), cu_b(cap_seqs + 1), bt(cap_blocks), pos(cap_tokens), slot(cap_tokens);
    for (int k = 0; k < 12; ++k) {
      cb_step st{};
      st.cap_seqs = cap_seqs; st.cap_tokens = cap_tokens; st.cap_blocks = cap_blocks;
      st.seq_ids = seq_ids.data(); st.cu_seqlens_q = cu_q.data(); st.context_lens = ctx.data(); st.cu_blocks = cu_b.data();
      st.block_table = bt.data(); st.positions = pos.data(); st.slot_mapping = slot.data();
      const int rc = cb_build_step(s, U(0, 700), &st);
      if (rc != CB_OK) { errs[3 + (-rc % 5)]++; }
      else {
        ++steps;
        // invariants the caller relies on
        if (st.num_tokens > cap_tokens || st.num_seqs > cap_seqs || st.num_blocks_emitted > cap_blocks) { printf("cap violated\n"); return 1; }
        if (cu_q[0] != 0 || cu_q[st.num_seqs] != st.num_tokens || cu_b[st.num_seqs] != st.num_blocks_emitted) { printf("prefix sums\n"); return 1; }
        for (int t = 0; t < st.num_tokens; ++t) if (slot[t] < 0 || slot[t] >= cfg.num_blocks * cfg.block_size) { printf("slot\n"); return 1; }
      }
      if (U(0, 4) == 0 && !ids.empty()) { cb_sched_finish(s, ids[U(0, (int)ids.size() - 1)]); }
      if (U(0, 6) == 0) { cb_sched* c = nullptr; if (cb_sched_clone(s, &c) == CB_OK) { cb_sched_destroy(s); s = c; } }
      if (U(0, 8) == 0) { int32_t id; int L = U(1, 500); if (cb_sched_add_prompt(s, L, 0, &id) == CB_OK) ids.push_back(id); }
      int32_t buf[64], n = 0;
      if (!ids.empty()) cb_sched_get_blocks(s, ids[U(0, (int)ids.size() - 1)], buf, 64, &n);
      int32_t np = 0, nf = 0; cb_sched_pending_prompts(s, &np); cb_sched_free_blocks(s, &nf);
    }
    cb_sched_destroy(s);
  }
  printf("ok: %d configs, %ld steps built; create-fail %ld run-fail %ld prompt-fail %ld step errs %ld %ld %ld %ld %ld\n",
         iters, steps, errs[0], errs[1], errs[2], errs[3], errs[4], errs[5], errs[6], errs[7]);
  return 0;
}
