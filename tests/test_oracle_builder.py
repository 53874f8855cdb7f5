"""Pins for the reference batch builder (oracle/builder.py) against what the pages fix.  CPU only."""
import itertools
import math

import pytest

from oracle.builder import BuildError, RefBuilder
from tests.conftest import golden


def _chunks_of(plan, rid):
    return [t for r, t in plan["prefill_chunks"] if r == rid]


def test_budget8_worked_example_matches_printed_table():
    g = golden("budget8_worked_example.json")
    b = RefBuilder(16, 64)
    for ctx in (16, 20, 24):
        b.add_running(ctx)
    p = b.add_prompt(g["prompt_len"])
    done = 0
    for rnd in g["rounds"]:
        plan = b.build(g["budget"])
        chunk = sum(_chunks_of(plan, p))
        assert plan["num_decodes"] == rnd["decode_tokens"]
        assert chunk == rnd["prompt_chunk"]
        done += chunk
        assert done == rnd["prompt_done"]
        assert plan["num_tokens"] == rnd["used"]
        assert plan["num_tokens"] + plan["unused_tokens"] == g["budget"]
    # round 4: P decodes at position 12, after D1..D3
    assert plan["decode_ids"][-1] == p and plan["positions"][-1] == 12


def test_chunk_tensors_of_round_two():
    g = golden("chunk_tensors_12_at_5.json")
    for bs in (4, 16):
        b = RefBuilder(bs, 64)
        p = b.add_prompt(g["prompt_len"])
        b.build(g["chunk_start"])                       # first round computes [0:5)
        plan = b.build(g["chunk_len"])                  # second round computes [5:10)
        assert plan["positions"] == g["positions"]
        assert plan["context_lens"] == [g["context_len_after_round"]]
        assert plan["cu_blocks"][-1] == math.ceil(g["context_len_after_round"] / bs)
        blocks = b.blocks_of(p)
        assert plan["slot_mapping"] == [blocks[q // bs] * bs + q % bs for q in g["positions"]]


def test_three_prompts_at_budget_2048_drain_in_four_iterations():
    # Derived by hand from the rule in §03 of "Chunked Prefill: Ending the Great Stall"
    # (12 decodes; prompts A 3072, B 2486, C 2580; budget 2048):
    #   it1: 12 decodes, A 2036                 it2: 12 decodes, A 1036 (done), B 1000
    #   it3: 13 decodes (A joined), B 1486 (done), C 549
    #   it4: 14 decodes (B joined), C 2031 (done), 3 tokens unused
    b = RefBuilder(16, 4096)
    for _ in range(12):
        b.add_running(100)
    A, B, C = b.add_prompt(3072), b.add_prompt(2486), b.add_prompt(2580)
    want = [(12, [(A, 2036)], 0), (12, [(A, 1036), (B, 1000)], 0),
            (13, [(B, 1486), (C, 549)], 0), (14, [(C, 2031)], 3)]
    for nd, chunks, unused in want:
        plan = b.build(2048)
        assert plan["num_decodes"] == nd
        assert plan["prefill_chunks"] == chunks
        assert plan["unused_tokens"] == unused
    assert b.pending_prompts() == 0


def test_prompt_4096_chunk_counts():
    g = golden("prompt4096_chunk_counts.json")
    for case in g["no_decodes"]:
        b = RefBuilder(16, 512)
        p = b.add_prompt(g["prompt_len"])
        n = 0
        while b.pending_prompts():
            plan = b.build(case["budget"])
            assert _chunks_of(plan, p) == [case["budget"]]
            n += 1
        assert n == case["chunks"]
    wd = g["with_decodes"]
    b = RefBuilder(16, 4096)
    for _ in range(wd["num_decodes"]):
        b.add_running(600)
    p = b.add_prompt(g["prompt_len"])
    sizes = []
    while b.pending_prompts():
        sizes.append(sum(_chunks_of(b.build(wd["budget"]), p)))
    assert sizes[:-1] == [wd["prefill_per_round"]] * (len(sizes) - 1)
    assert sizes == [448] * 9 + [64]


def test_prefix_reread_closed_form():
    g = golden("prefix_reread.json")
    b = RefBuilder(16, 512)
    b.add_prompt(g["prompt_len"])
    reads = 0
    steps = 0
    while b.pending_prompts():
        plan = b.build(g["chunk"])
        reads += plan["context_lens"][0]                # chunk k reads the KV of k chunks
        steps += 1
    C, N = g["chunk"], g["chunks"]
    assert steps == N
    assert reads == C * N * (N + 1) // 2 == g["kv_token_reads_chunked"]
    assert round(reads / g["kv_token_reads_monolithic"], 1) == g["ratio_approx"]


def test_attention_pairs_do_not_depend_on_the_split():
    # Splitting Prefill From Decode Inside a Step, "The arithmetic of chunk boundaries": causal
    # attention is about T^2/2 pairs however the prompt is cut.  Exactly: sum of (pos+1) = T(T+1)/2.
    for budget in (1, 7, 448, 512, 5000):
        b = RefBuilder(16, 512)
        b.add_prompt(4096)
        pairs = 0
        while b.pending_prompts():
            pairs += sum(p + 1 for p in b.build(budget)["positions"])
        assert pairs == 4096 * 4097 // 2


def test_exercise_budget16_six_decodes_two_prompts():
    # Chunked Prefill 的 Token 预算 §16, first exercise, derived by hand:
    #   r1: 6 decodes, P1 10       r2: 6 decodes, P1 8 (done), P2 2       r3: 7 decodes, P2 3
    b = RefBuilder(16, 256)
    for _ in range(6):
        b.add_running(30)
    P1, P2 = b.add_prompt(18), b.add_prompt(5)
    want = [(6, [(P1, 10)], 16), (6, [(P1, 8), (P2, 2)], 16), (7, [(P2, 3)], 10)]
    for nd, chunks, used in want:
        plan = b.build(16)
        assert (plan["num_decodes"], plan["prefill_chunks"], plan["num_tokens"]) == (nd, chunks, used)


def test_exercise_split_4_3_3_positions_and_context():
    # §16, second exercise: prompt of 10 in chunks [4, 3, 3].
    b = RefBuilder(16, 16)
    b.add_prompt(10)
    got = [b.build(t) for t in (4, 3, 3)]
    assert [g["positions"] for g in got] == [[0, 1, 2, 3], [4, 5, 6], [7, 8, 9]]
    assert [g["context_lens"] for g in got] == [[4], [7], [10]]


def test_decodes_over_budget_is_an_error_and_changes_nothing():
    b = RefBuilder(16, 64)
    for _ in range(5):
        b.add_running(16)
    b.add_prompt(20)
    snap = b.clone()
    with pytest.raises(BuildError) as e:
        b.build(4)
    assert e.value.reason == "decode_over_budget"
    assert b.__dict__.keys() == snap.__dict__.keys()
    assert list(b.free) == list(snap.free) and b.running == snap.running and b.waiting == snap.waiting
    plan = b.build(5)                                 # exactly the decodes, no chunk
    assert plan["num_decodes"] == 5 and plan["prefill_chunks"] == [] and plan["unused_tokens"] == 0


def test_decode_growth_out_of_blocks_is_atomic():
    b = RefBuilder(4, 2)
    b.add_running(4)                                  # one full block
    b.add_running(4)                                  # the other
    snap = b.clone()
    with pytest.raises(BuildError) as e:
        b.build(8)
    assert e.value.reason == "out_of_blocks"
    assert b.running == snap.running and list(b.free) == list(snap.free)


def test_full_prompt_reservation_and_strict_fcfs():
    b = RefBuilder(4, 5)
    b.add_running(3)                                  # 1 block, room for one more token
    P1 = b.add_prompt(12)                             # needs 3 blocks
    P2 = b.add_prompt(2)                              # needs 1 block
    plan = b.build(3)                                 # 1 decode + 2 tokens of P1; P1 reserves 3
    assert plan["prefill_chunks"] == [(P1, 2)]
    assert len(b.blocks_of(P1)) == 3 and len(b.free) == 1
    b2 = RefBuilder(4, 3)
    b2.add_running(3)
    Q1 = b2.add_prompt(12)                            # 3 blocks > 2 free: head cannot be reserved
    b2.add_prompt(2)
    plan = b2.build(8)
    assert plan["prefill_chunks"] == [] and plan["unused_tokens"] == 7   # no skipping
    assert len(b2.blocks_of(Q1)) == 0


def test_cached_prefix_computes_only_the_suffix():
    b = RefBuilder(32, 64)
    p = b.add_prompt(100, cached_len=70)
    assert len(b.blocks_of(p)) == 3
    plan = b.build(1000)
    assert plan["positions"] == list(range(70, 100))
    assert plan["context_lens"] == [100] and plan["unused_tokens"] == 970
    assert len(b.blocks_of(p)) == 4


def test_invalid_requests():
    b = RefBuilder(16, 8)
    for args in [(0,), (5, 5), (5, -1), (5, 6)]:
        with pytest.raises(BuildError):
            b.add_prompt(*args)
    with pytest.raises(BuildError):
        b.add_running(0)
    with pytest.raises(BuildError):
        b.build(0)


def test_chunk_cap_off_by_default_and_capping_when_set():
    b = RefBuilder(16, 64, max_chunk=4)
    P1, P2 = b.add_prompt(10), b.add_prompt(3)
    plan = b.build(16)
    assert plan["prefill_chunks"] == [(P1, 4), (P2, 3)]


def test_prefill_starvation_when_decodes_fill_the_budget():
    # §08 of the zwjcode page: strict decode-first can starve a prompt when decodes fill the budget.
    b = RefBuilder(16, 256)
    for _ in range(4):
        b.add_running(10)
    b.add_prompt(5)
    for _ in range(20):
        assert b.build(4)["prefill_chunks"] == []
    assert b.pending_prompts() == 1


def _check_invariants(plan, budget, bs, history, running_before):
    cu = plan["cu_seqlens_q"]
    assert plan["num_tokens"] <= budget
    assert plan["num_tokens"] + plan["unused_tokens"] == budget
    qlens = [cu[i + 1] - cu[i] for i in range(plan["num_seqs"])]
    assert all(q > 0 for q in qlens)
    nd = plan["num_decodes"]
    assert all(q == 1 for q in qlens[:nd])
    assert plan["decode_ids"] == running_before or plan["decode_ids"][:len(running_before)] == running_before
    for s in range(plan["num_seqs"]):
        rid = plan["seq_ids"][s]
        pos = plan["positions"][cu[s]:cu[s + 1]]
        assert pos == list(range(pos[0], pos[0] + len(pos)))          # contiguous
        assert plan["context_lens"][s] == pos[-1] + 1
        blocks = plan["block_table"][plan["cu_blocks"][s]:plan["cu_blocks"][s + 1]]
        assert len(blocks) == -(-plan["context_lens"][s] // bs)
        for p, sl in zip(pos, plan["slot_mapping"][cu[s]:cu[s + 1]]):
            assert sl == blocks[p // bs] * bs + p % bs
        if s >= nd:                                                     # chunk: no overlap
            prev = history.setdefault(rid, 0)
            assert pos[0] == prev
            history[rid] = pos[-1] + 1
    slots = plan["slot_mapping"]
    assert len(set(slots)) == len(slots)                               # no slot written twice


def test_invariants_exhaustive_small():
    # Every budget 1..8, up to 3 prompts of length 1..10 (a subset of lengths), 0..2 decodes.
    lengths = [1, 2, 5, 7, 10]
    for budget in range(1, 9):
        for nd in range(0, 3):
            for k in range(1, 4):
                for lens in itertools.product(lengths, repeat=k):
                    b = RefBuilder(4, 128)
                    for _ in range(nd):
                        b.add_running(3)
                    rids = [b.add_prompt(L) for L in lens]
                    hist = {}
                    steps = 0
                    while b.pending_prompts():
                        next_decodes = len(b.running) + sum(w.done == w.length for w in b.waiting)
                        if next_decodes >= budget:
                            break                   # decodes fill the budget: prompts starve
                        before = [r.rid for r in b.running]
                        plan = b.build(budget)
                        _check_invariants(plan, budget, 4, hist, before)
                        # leftover budget only when nothing else could be scheduled
                        if plan["unused_tokens"] > 0:
                            assert b.pending_prompts() == 0
                        steps += 1
                        assert steps < 200
                    if b.pending_prompts() == 0:
                        for rid, L in zip(rids, lens):
                            assert hist[rid] == L


# ---------------------------------------------------------------------------------------------
# Caps and priority policies.
# ---------------------------------------------------------------------------------------------
from oracle.builder import DECODE_FIRST, FAIR_SHARE, PREFILL_FIRST  # noqa: E402


def test_threshold_ceiling_gives_budget_over_threshold_partial_prefills():
    # The sference.com post, "The fix": dividing the round's budget by the per-request threshold
    # gives the number of partial prefills run at once: 8192 // 4096 = 2, 16384 // 4096 = 4.
    for budget, want in ((8192, 2), (16384, 4)):
        b = RefBuilder(16, 40000, max_chunk=4096)
        rids = [b.add_prompt(100000) for _ in range(6)]
        plan = b.build(budget)
        assert plan["prefill_chunks"] == [(r, 4096) for r in rids[:want]]
        assert plan["unused_tokens"] == 0


def test_threshold_ceiling_idles_a_lone_long_prompt_and_the_floor_does_not():
    # The same post, caveats and closing section: with the ceiling a lone long request is capped
    # at the threshold and the rest of the budget idles; with the proposed floor one long prefill on
    # its own takes all of the budget and two take half each.
    ceil_b = RefBuilder(16, 40000, max_chunk=4096)
    ceil_b.add_prompt(100000)
    plan = ceil_b.build(8192)
    assert plan["num_prefill_tokens"] == 4096 and plan["unused_tokens"] == 4096
    floor_b = RefBuilder(16, 40000, prefill_floor=4096)
    floor_b.add_prompt(100000)
    plan = floor_b.build(8192)
    assert plan["num_prefill_tokens"] == 8192 and plan["unused_tokens"] == 0
    for floor in (1024, 2048, 4096):
        two = RefBuilder(16, 40000, prefill_floor=floor)
        a, c = two.add_prompt(100000), two.add_prompt(100000)
        assert two.build(8192)["prefill_chunks"] == [(a, 4096), (c, 4096)]


def test_floor_keeps_short_prompts_whole_and_shares_the_rest_evenly():
    # Short prompts (at most the floor) are admitted whole; the long ones get at least the floor
    # and split what is left evenly; an odd token goes to the first of them.
    b = RefBuilder(16, 40000, prefill_floor=1000)
    L1, S1, L2, S2 = b.add_prompt(50000), b.add_prompt(300), b.add_prompt(50000), b.add_prompt(700)
    plan = b.build(5001)
    # first pass: 1000 + 300 + 1000 + 700 = 3000; 2001 left, split 1001 / 1000 between L1 and L2
    assert plan["prefill_chunks"] == [(L1, 2001), (S1, 300), (L2, 2000), (S2, 700)]


def test_threshold_removes_head_of_line_blocking():
    # The sference.com post, "One slot, one request": a cold 600,000-token prompt is followed by four
    # small prompts and two 300,000-token prompts with a 99% cache hit.  Admitted whole, the big
    # prompt holds the round's budget until it is done (74 rounds of 8192) and all six wait behind
    # it; with the 4096-token threshold they all finish their prefill within the first rounds.
    def first_token_rounds(max_chunk):
        b = RefBuilder(64, 40000, max_chunk=max_chunk)
        b.add_prompt(600000)
        small = [b.add_prompt(2000) for _ in range(4)]
        cached = [b.add_prompt(300000, 297000) for _ in range(2)]
        done = {}
        for rnd in range(1, 80):
            plan = b.build(8192)
            for w in b.waiting:
                if w.done == w.length and w.rid not in done:
                    done[w.rid] = rnd
            if all(r in done for r in small + cached):
                break
        return [done.get(r) for r in small + cached]
    # Admitted whole (by hand): rounds 1-73 give the big prompt 8192 each; round 74 its last 1984
    # and then 2000 to each of the first three small prompts and 208 to the fourth; round 75 (the
    # big one now decodes) finishes the fourth and both cached prompts.
    assert first_token_rounds(0) == [74, 74, 74, 75, 75, 75]
    # With the threshold (by hand): round 1 big 4096, small 2000 + 2000 + 96; round 2 big 4096,
    # small 1904 (done) + 2000, cached 192; round 3 big 4096, cached 2808 (done) + 1288; round 4
    # big 4096, cached 1712 (done).
    assert first_token_rounds(4096) == [1, 1, 2, 2, 3, 4]


def test_partial_prefill_cap_skips_only_prompts_that_would_stay_unfinished():
    b = RefBuilder(16, 4096, max_chunk=30, max_partial_prefills=1)
    p0, p1, p2, p3 = b.add_prompt(200), b.add_prompt(200), b.add_prompt(20), b.add_prompt(200)
    plan = b.build(100)
    assert plan["prefill_chunks"] == [(p0, 30), (p2, 20)]
    assert plan["unused_tokens"] == 50


def test_sequence_cap_limits_chunks_and_rejects_too_many_strict_decodes():
    b = RefBuilder(16, 4096, max_num_seqs=5)
    for _ in range(4):
        b.add_running(10)
    p0, p1 = b.add_prompt(100), b.add_prompt(100)
    plan = b.build(64)
    assert plan["num_seqs"] == 5 and plan["prefill_chunks"] == [(p0, 60)]
    over = RefBuilder(16, 4096, max_num_seqs=3)
    for _ in range(4):
        over.add_running(10)
    with pytest.raises(BuildError) as e:
        over.build(64)
    assert e.value.reason == "decode_over_budget"


def test_prefill_quota_lets_a_prompt_finish_beside_decodes_that_never_drain():
    # "Chunked Prefill 的 Token 预算" §16, third exercise: reserve at least 25% of every round for
    # prefill, build traffic whose decodes never empty, and check the long prompt still finishes.
    # Budget 16 with 16 decodes: strict decode-first never schedules the prompt; with the quota,
    # decodes use at most 12 tokens, the prompt gets 4 per round and finishes in 40 / 4 rounds, and
    # with 12 decode slots for 16 decodes each decode runs at least every second round.
    strict = RefBuilder(16, 4096)
    quota = RefBuilder(16, 4096, prefill_quota_pct=25)
    for b in (strict, quota):
        for _ in range(16):
            b.add_running(10)
        b.add_prompt(40)
    for _ in range(30):
        assert strict.build(16)["prefill_chunks"] == []
    ran = []
    for rnd in range(10):
        plan = quota.build(16)
        assert plan["num_decodes"] == 12 and plan["num_prefill_tokens"] == 4
        ran.append(set(plan["decode_ids"]))
    assert quota.pending_prompts() == 0
    for a, c in zip(ran, ran[1:]):
        assert a | c == set(range(16))
    # prompt done: its first decode (round 11) competes like any other; no prompt waits, so the
    # quota no longer holds anything back and all 17 decodes fit a budget of 17
    assert quota.build(17)["num_decodes"] == 17


def test_priority_policies_split_the_budget_as_named():
    # "Splitting Prefill From Decode Inside a Step", "Choosing the priority order".
    def run(policy, **kw):
        b = RefBuilder(16, 4096, policy=policy, **kw)
        for _ in range(4):
            b.add_running(10)
        b.add_prompt(100)
        return b.build(16)
    df = run(DECODE_FIRST)
    assert (df["num_decodes"], df["num_prefill_tokens"]) == (4, 12)
    pf = run(PREFILL_FIRST)                      # prompts take the budget, decodes get nothing
    assert (pf["num_decodes"], pf["num_prefill_tokens"]) == (0, 16)
    fs = run(FAIR_SHARE, decode_share_pct=50)    # decodes need 4 of their 8: prompts get 12
    assert (fs["num_decodes"], fs["num_prefill_tokens"]) == (4, 12)
    fs2 = run(FAIR_SHARE, decode_share_pct=10)   # decodes' share ceil(1.6) = 2; 14 to the prompt
    assert (fs2["num_decodes"], fs2["num_prefill_tokens"]) == (2, 14)


def test_prefill_first_runs_decodes_in_the_budget_the_prompts_leave():
    b = RefBuilder(16, 4096, policy=PREFILL_FIRST)
    for _ in range(4):
        b.add_running(10)
    p = b.add_prompt(10)
    plan = b.build(16)
    assert plan["prefill_chunks"] == [(p, 10)] and plan["num_decodes"] == 4
    assert plan["unused_tokens"] == 2


def test_deferred_decodes_run_longest_waiting_first():
    b = RefBuilder(16, 4096, policy=FAIR_SHARE, decode_share_pct=25)
    ids = [b.add_running(10) for _ in range(6)]
    b.add_prompt(1000)
    seen = [b.build(8)["decode_ids"] for _ in range(3)]     # 2 decode slots per round
    assert seen == [ids[0:2], ids[2:4], ids[4:6]]


def test_finish_returns_blocks_to_the_back_of_the_pool():
    b = RefBuilder(4, 10)
    d = b.add_running(6)                 # blocks 0, 1
    p = b.add_prompt(3)                  # no cached blocks yet
    b.build(8)                           # d grows? position 6 fits block 1; p reserves block 2
    assert b.blocks_of(d) == [0, 1] and b.blocks_of(p) == [2]
    with pytest.raises(BuildError):
        b.finish(99)
    b.finish(d)
    assert list(b.free) == [3, 4, 5, 6, 7, 8, 9, 0, 1]
    b.finish(p)                          # its last chunk has run: it may finish before decoding
    assert list(b.free)[-1] == 2
    q = b.add_prompt(5)
    with pytest.raises(BuildError):
        b.finish(q)                      # tokens still to compute
