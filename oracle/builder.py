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


@dataclasses.dataclass
class _Waiting:
    rid: int
    length: int         # prompt length L
    done: int           # tokens whose K/V are already in the cache (cached prefix + chunks run)
    blocks: list
    reserved: bool


class RefBuilder:
    """Block pool + running/waiting queues + the per-step build."""

    def __init__(self, block_size: int, num_blocks: int, free_list=None, max_chunk: int = 0):
        if block_size < 1 or num_blocks < 0 or max_chunk < 0:
            raise BuildError("invalid", "bad pool geometry")
        order = list(range(num_blocks)) if free_list is None else [int(b) for b in free_list]
        if sorted(order) != list(range(num_blocks)):
            raise BuildError("invalid", "free list must be a permutation of the pool")
        self.bs = block_size
        self.max_chunk = max_chunk
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

    # ---- one step ----------------------------------------------------------------------
    def build(self, budget: int) -> dict:
        """Plan one mixed step under ``budget`` tokens and commit it; see the module docstring."""
        if budget < 1:
            raise BuildError("invalid", "token budget must be >= 1")
        bs = self.bs
        free = collections.deque(self.free)
        running = [_Running(r.rid, r.ctx, list(r.blocks)) for r in self.running]
        waiting = []
        for w in self.waiting:                        # graduation: finished prompts decode now
            w = _Waiting(w.rid, w.length, w.done, list(w.blocks), w.reserved)
            if w.done == w.length:
                running.append(_Running(w.rid, w.length, w.blocks))
            else:
                waiting.append(w)
        if len(running) > budget:
            raise BuildError("decode_over_budget", f"{len(running)} decodes > budget {budget}")

        seqs = []   # (rid, first position, number of query tokens, blocks list)
        for r in running:                             # decode-maximal: every running request
            pos = r.ctx
            if pos == bs * len(r.blocks):
                r.blocks.extend(self._take_blocks(free, 1))
            seqs.append((r.rid, pos, 1, r.blocks))
            r.ctx += 1
        left = budget - len(running)

        chunks = []
        for w in waiting:                             # FCFS walk over the leftover budget
            if left == 0:
                break
            if not w.reserved:
                need = _ceil_div(w.length, bs) - len(w.blocks)
                if need > len(free):
                    break                             # strict FCFS: the head waits for blocks
                w.blocks.extend(self._take_blocks(free, need))
                w.reserved = True
            take = min(w.length - w.done, left)
            if self.max_chunk:
                take = min(take, self.max_chunk)
            seqs.append((w.rid, w.done, take, w.blocks))
            chunks.append((w.rid, take))
            w.done += take
            left -= take

        plan = self._emit(seqs, len(running), budget, left)
        plan["decode_ids"] = [r.rid for r in running]
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
