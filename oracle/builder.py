"""Reference batch builder for one mixed step (oracle; test infrastructure only).

What it follows:

* Chunked Prefill: Ending the Great Stall (manishklach), §03 "Chunked prefill mechanics" and §04
  "Stall-free scheduling": every running decode is placed first at one token each; the waiting
  prompts are then walked in order and each gets the largest chunk that fits what is left of the
  budget; a prompt that does not fit gets a smaller chunk and continues next iteration; a prompt
  whose last chunk ran joins the decode set.
* Chunked Prefill 的 Token 预算 (zwjcode), §04 (the budget inequality |D_t| + sum|c| <= B_tok),
  §05 (the teaching scheduler: error when decodes exceed the budget, FCFS walk, take =
  min(remaining, budget left), report of decode ids / chunks / unused tokens), §06 (per-chunk
  positions, slot_mapping, block_table of ceil(context/B) entries, context length after the
  round), §08 (decodes first, then prefill, then one step, then an atomic commit) and §11 (KV
  blocks are reserved for the whole input sequence at admission).
* Splitting Prefill From Decode Inside a Step (mercemay), "The arithmetic of chunk boundaries":
  the cache must be reserved before the first chunk; "Chunked prefill as a rate control": the
  optional per-prefill chunk cap (off by default).

Readings taken where the pages are silent (each also listed in the design notes): decodes over
budget is an error and nothing changes; a finished prompt decodes from the next step on, placed
after the existing decodes, its first decode position being its length; rows are ordered decodes
first (running order) then chunks (FCFS order); a decode with context L has L tokens cached, so its
query sits at position L and its emitted context length is L + 1; blocks come off the front of the
caller's free list; a prompt's whole length is reserved when it first gets tokens, and if the head
of the queue cannot be reserved the walk stops there (no skipping); a decode that needs a new
block when none is free is an error (no preemption); the block table is ragged with exactly
ceil(context_len / block_size) entries per sequence; state changes only when a build succeeds.

Optional caps and policies (all off by default, and then the build is the one above):

* Per-request cap ``max_chunk``: "Splitting Prefill From Decode Inside a Step" caps a prefill's
  take at its chunk size; the sference.com post's shipped long-prefill threshold ("The fix") is the
  same ceiling (no request takes more than the threshold per round).
* ``prefill_floor``: the sference.com post's proposed floor (closing section): a long prompt is
  guaranteed up to the floor per round and expands into whatever budget is left. Reading: a first
  FCFS pass grants min(remaining, floor, left) to each admitted prompt; the budget left after it
  is then shared evenly among the admitted prompts that still have tokens (each bounded by its
  remaining tokens and the per-request cap), an indivisible rest going one token each in FCFS
  order. One long prompt alone takes the whole budget; two take half each.
* ``max_partial_prefills`` and ``max_num_seqs`` ("Chunked Prefill 的 Token 预算" §10: at most
  that many prompts partly prefilled at once; at most that many sequences per step). Readings: a
  prompt whose first-pass grant leaves it unfinished is admitted only while fewer than
  ``max_partial_prefills`` admitted prompts stay unfinished, else it is skipped this step (prompts
  behind it that finish within the step may still be admitted); the prompt walk stops when the
  step holds ``max_num_seqs`` sequences.
* ``policy`` ("Splitting Prefill From Decode Inside a Step", "Choosing the priority order"):
  decode-first (the default above), prefill-first (the prompt walk gets the whole budget, decodes
  run in what is left) and fair share (decodes get up to ``decode_share_pct`` of the budget, the
  prompts the rest, each class's unused share going to the other). ``prefill_quota_pct``
  ("Chunked Prefill 的 Token 预算" §08 and §16: reserve part of each round for prefill so that a
  decode batch that never drains cannot starve prompts): under decode-first, while prompts wait,
  decodes use at most the budget minus that share. Under these policies (and a sequence cap) a
  decode that does not fit waits for a later step instead of failing; the ones that have waited
  longest run first (running order breaks ties), and the decodes that run are emitted in running
  order. Under plain decode-first, decodes beyond the budget or the sequence cap are an error as
  above.
* ``finish(rid)`` retires a request that has produced its last token (a running decode, or a
  prompt whose last chunk has run) and returns its blocks to the back of the free list.
"""
from __future__ import annotations

import collections
import copy
import dataclasses


class BuildError(Exception):
    """A build or setup request that the builder refuses; ``reason`` names the case."""

    def __init__(self, reason: str, msg: str = ""):
        super().__init__(f"{reason}: {msg}" if msg else reason)
        self.reason = reason


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclasses.dataclass
class _Running:
    rid: int
    ctx: int            # tokens in the cache
    blocks: list
    waited: int = 0     # consecutive steps this decode did not run


@dataclasses.dataclass
class _Waiting:
    rid: int
    length: int         # prompt length L
    done: int           # tokens whose K/V are already in the cache (cached prefix + chunks run)
    blocks: list
    reserved: bool


DECODE_FIRST, PREFILL_FIRST, FAIR_SHARE = 0, 1, 2


class RefBuilder:
    """Block pool + running/waiting queues + the per-step build."""

    def __init__(self, block_size: int, num_blocks: int, free_list=None, max_chunk: int = 0,
                 prefill_floor: int = 0, max_partial_prefills: int = 0, max_num_seqs: int = 0,
                 policy: int = DECODE_FIRST, decode_share_pct: int = 0, prefill_quota_pct: int = 0):
        if block_size < 1 or num_blocks < 0 or max_chunk < 0:
            raise BuildError("invalid", "bad pool geometry")
        if (prefill_floor < 0 or max_partial_prefills < 0 or max_num_seqs < 0
                or policy not in (DECODE_FIRST, PREFILL_FIRST, FAIR_SHARE)
                or not 0 <= decode_share_pct <= 99 or not 0 <= prefill_quota_pct <= 100):
            raise BuildError("invalid", "bad cap or policy")
        order = list(range(num_blocks)) if free_list is None else [int(b) for b in free_list]
        if sorted(order) != list(range(num_blocks)):
            raise BuildError("invalid", "free list must be a permutation of the pool")
        self.bs = block_size
        self.max_chunk = max_chunk
        self.prefill_floor = prefill_floor
        self.max_partial = max_partial_prefills
        self.max_seqs = max_num_seqs
        self.policy = policy
        self.decode_share_pct = decode_share_pct or 50
        self.quota_pct = prefill_quota_pct
        self.free = collections.deque(order)
        self.running: list[_Running] = []
        self.waiting: list[_Waiting] = []
        self.next_id = 0

    # ---- setup -------------------------------------------------------------------------
    def _take_blocks(self, free, n: int):
        if n > len(free):
            raise BuildError("out_of_blocks", f"need {n}, have {len(free)}")
        return [free.popleft() for _ in range(n)]

    def add_running(self, context_len: int) -> int:
        """A request already decoding, with ``context_len`` tokens in the cache."""
        if context_len < 1:
            raise BuildError("invalid", "a decode needs at least one cached token")
        blocks = self._take_blocks(self.free, _ceil_div(context_len, self.bs))
        rid = self.next_id
        self.next_id += 1
        self.running.append(_Running(rid, context_len, blocks))
        return rid

    def add_prompt(self, prompt_len: int, cached_len: int = 0) -> int:
        """A prompt of ``prompt_len`` tokens whose first ``cached_len`` are already cached."""
        if prompt_len < 1 or cached_len < 0 or cached_len > prompt_len - 1:
            raise BuildError("invalid", "need prompt_len >= 1 and 0 <= cached_len < prompt_len")
        blocks = self._take_blocks(self.free, _ceil_div(cached_len, self.bs))
        rid = self.next_id
        self.next_id += 1
        self.waiting.append(_Waiting(rid, prompt_len, cached_len, blocks, False))
        return rid

    def blocks_of(self, rid: int) -> list:
        for r in self.running:
            if r.rid == rid:
                return list(r.blocks)
        for w in self.waiting:
            if w.rid == rid:
                return list(w.blocks)
        raise BuildError("invalid", f"unknown request {rid}")

    def clone(self) -> "RefBuilder":
        return copy.deepcopy(self)

    def finish(self, rid: int) -> None:
        """Retire a request that produced its last token; its blocks go to the back of the pool."""
        for i, r in enumerate(self.running):
            if r.rid == rid:
                self.free.extend(r.blocks)
                del self.running[i]
                return
        for i, w in enumerate(self.waiting):
            if w.rid == rid and w.done == w.length:
                self.free.extend(w.blocks)
                del self.waiting[i]
                return
        raise BuildError("invalid", f"request {rid} has not produced a token")

    # ---- one step ----------------------------------------------------------------------
    def build(self, budget: int) -> dict:
        """Plan one mixed step under ``budget`` tokens and commit it; see the module docstring."""
        if budget < 1:
            raise BuildError("invalid", "token budget must be >= 1")
        bs = self.bs
        free = collections.deque(self.free)
        running = [_Running(r.rid, r.ctx, list(r.blocks), r.waited) for r in self.running]
        waiting = []
        for w in self.waiting:                        # graduation: finished prompts decode now
            w = _Waiting(w.rid, w.length, w.done, list(w.blocks), w.reserved)
            if w.done == w.length:
                running.append(_Running(w.rid, w.length, w.blocks))
            else:
                waiting.append(w)
        nd_all = len(running)
        seq_cap = self.max_seqs or (nd_all + len(waiting))
        prompts_wait = len(waiting) > 0

        # How many decodes may run, by policy.
        strict = self.policy == DECODE_FIRST and self.quota_pct == 0
        if strict:
            if nd_all > budget:
                raise BuildError("decode_over_budget", f"{nd_all} decodes > budget {budget}")
            if nd_all > seq_cap:
                raise BuildError("decode_over_budget", f"{nd_all} decodes > sequence cap {seq_cap}")
            dec_limit = nd_all
        elif self.policy == DECODE_FIRST:
            reserve = -(-self.quota_pct * budget // 100) if prompts_wait else 0
            dec_limit = min(nd_all, budget - reserve, seq_cap)
        elif self.policy == FAIR_SHARE:
            dec_limit = min(nd_all, -(-self.decode_share_pct * budget // 100), seq_cap)
        else:                                         # prefill-first: decodes come after the walk
            dec_limit = 0

        # The decodes that run: longest-waiting first, running order among equals.
        order = sorted(range(nd_all), key=lambda i: (-running[i].waited, i))
        chosen = set(order[:dec_limit])
        left = budget - len(chosen)
        nseq = len(chosen)
        # Blocks the chosen decodes need come before any prompt's reservation; a decode that
        # cannot grow is an error (no preemption).
        free_avail = len(free) - sum(1 for i in chosen if running[i].ctx == bs * len(running[i].blocks))
        if free_avail < 0:
            raise BuildError("out_of_blocks", "a decode needs a new block")

        # Prompt walk, first pass (FCFS).
        grants = []          # [waiting index, tokens, blocks to reserve]
        partial = 0
        for wi, w in enumerate(waiting):
            if left == 0 or nseq >= seq_cap:
                break
            rem = w.length - w.done
            g = min(rem, left)
            if self.max_chunk:
                g = min(g, self.max_chunk)
            if self.prefill_floor:
                g = min(g, self.prefill_floor)
            if self.max_partial and g < rem and partial >= self.max_partial:
                continue                              # would stay unfinished past the cap
            need = 0
            if not w.reserved:
                need = _ceil_div(w.length, bs) - len(w.blocks)
                if need > free_avail:
                    break                             # strict FCFS: the head waits for blocks
                free_avail -= need
            grants.append([wi, g, need])
            partial += g < rem
            nseq += 1
            left -= g
        # Floor: the budget left is shared evenly among the admitted prompts with tokens to go.
        if self.prefill_floor:
            def room(gr):
                w = waiting[gr[0]]
                top = w.length - w.done
                if self.max_chunk:
                    top = min(top, self.max_chunk)
                return top - gr[1]
            while left > 0:
                active = [gr for gr in grants if room(gr) > 0]
                if not active:
                    break
                share = left // len(active)
                if share == 0:
                    for gr in active[:left]:
                        gr[1] += 1
                    left = 0
                    break
                for gr in active:
                    d = min(room(gr), share)
                    gr[1] += d
                    left -= d
        # Decodes that did not get their turn take what the prompts left (every mode but plain
        # decode-first, where all of them already run).
        if not strict and left > 0:
            extra = min(nd_all - len(chosen), left, seq_cap - nseq)
            order = sorted(range(nd_all), key=lambda i: (-running[i].waited, i))
            add = [i for i in order if i not in chosen][:extra]
            free_avail -= sum(1 for i in add if running[i].ctx == bs * len(running[i].blocks))
            if free_avail < 0:
                raise BuildError("out_of_blocks", "a decode needs a new block")
            chosen |= set(add)
            nseq += len(add)
            left -= len(add)

        seqs = []   # (rid, first position, number of query tokens, blocks list)
        for i, r in enumerate(running):               # the decodes that run, in running order
            if i not in chosen:
                r.waited += 1
                continue
            r.waited = 0
            pos = r.ctx
            if pos == bs * len(r.blocks):
                r.blocks.extend(self._take_blocks(free, 1))
            seqs.append((r.rid, pos, 1, r.blocks))
            r.ctx += 1
        num_decodes = len(seqs)
        chunks = []
        for wi, g, need in grants:                    # then the chunks, in FCFS order
            w = waiting[wi]
            if not w.reserved:
                w.blocks.extend(self._take_blocks(free, need))
                w.reserved = True
            seqs.append((w.rid, w.done, g, w.blocks))
            chunks.append((w.rid, g))
            w.done += g

        plan = self._emit(seqs, num_decodes, budget, left)
        plan["decode_ids"] = [r.rid for i, r in enumerate(running) if i in chosen]
        plan["prefill_chunks"] = chunks
        self.free, self.running, self.waiting = free, running, waiting   # atomic commit
        return plan

    def _emit(self, seqs, num_decodes: int, budget: int, unused: int) -> dict:
        bs = self.bs
        seq_ids, cu_q, ctx_lens, cu_blocks, block_table = [], [0], [], [0], []
        positions, slots = [], []
        for rid, first, n, blocks in seqs:
            ctx = first + n                           # context length after the round
            seq_ids.append(rid)
            cu_q.append(cu_q[-1] + n)
            ctx_lens.append(ctx)
            nb = _ceil_div(ctx, bs)
            block_table.extend(blocks[:nb])
            cu_blocks.append(cu_blocks[-1] + nb)
            for p in range(first, first + n):         # absolute positions, never reset
                positions.append(p)
                slots.append(blocks[p // bs] * bs + p % bs)
        q_lens = [cu_q[i + 1] - cu_q[i] for i in range(len(seqs))]
        return {
            "seq_ids": seq_ids, "cu_seqlens_q": cu_q, "context_lens": ctx_lens,
            "cu_blocks": cu_blocks, "block_table": block_table,
            "positions": positions, "slot_mapping": slots,
            "num_seqs": len(seqs), "num_decodes": num_decodes, "num_tokens": cu_q[-1],
            "num_prefill_tokens": cu_q[-1] - num_decodes, "unused_tokens": unused,
            "max_q_len": max(q_lens, default=0), "max_context_len": max(ctx_lens, default=0),
            "num_blocks_emitted": len(block_table), "budget": budget,
        }

    # ---- queries used by tests ---------------------------------------------------------
    def pending_prompts(self) -> int:
        """Prompts that still have tokens to prefill."""
        return sum(1 for w in self.waiting if w.done < w.length)
