"""Reference step simulation over the reference builder (oracle; test infrastructure only).

Plain restatement of the bookkeeping the simulator follows: requests join the queue at their
arrival step; the step that runs a prompt's last chunk gives the request its first token ("Chunked
Prefill 的 Token 预算" §03: a finished prompt becomes a decode); each decode row gives one more;
a request with all its output tokens is retired and its blocks return to the pool.  Time to first
token = first-token step - arrival + 1; time between tokens = the step gap between consecutive
tokens of one request.
"""
from __future__ import annotations

from oracle.builder import BuildError, RefBuilder


def simulate(stream, budget, steps, running=(), block_size=16, num_blocks=1 << 16, **cfg):
    """``running``: (context_len, output_len) of requests decoding before step 1 (their indices
    follow the stream's)."""
    b = RefBuilder(block_size, num_blocks, **cfg)
    index, computed, tokens_out, last = {}, {}, {}, {}
    want = [r.output_len for r in stream] + [o for _, o in running]
    for j, (ctx, _) in enumerate(running):
        rid = b.add_running(ctx)
        index[rid], tokens_out[rid], last[rid] = len(stream) + j, 0, 0
    ttft, gaps = {}, []
    finished = used = idle = 0
    stop = ""
    pending = list(stream)
    step = 0
    for step in range(1, steps + 1):
        while pending and pending[0].arrival <= step:
            r = pending.pop(0)
            rid = b.add_prompt(r.prompt_len, r.cached_len)
            index[rid] = len(stream) - len(pending) - 1
            computed[rid] = r.cached_len
            tokens_out[rid] = 0
        try:
            plan = b.build(budget)
        except BuildError as e:
            stop = e.reason
            break
        used += plan["num_tokens"]
        idle += plan["unused_tokens"]
        retire = []
        for rid in plan["decode_ids"]:
            gaps.append(step - last[rid])
            last[rid] = step
            tokens_out[rid] += 1
            if tokens_out[rid] == want[index[rid]]:
                retire.append(rid)
        for rid, n in plan["prefill_chunks"]:
            computed[rid] += n
            r = stream[index[rid]]
            if computed[rid] == r.prompt_len:
                ttft[index[rid]] = step - r.arrival + 1
                last[rid] = step
                tokens_out[rid] += 1
                if tokens_out[rid] == want[index[rid]]:
                    retire.append(rid)
        for rid in retire:
            b.finish(rid)
            finished += 1
        if not pending and finished == len(want):
            break
    return {"steps": step, "ttft": ttft, "tbt": gaps, "finished": finished, "tokens": used,
            "unused": idle, "stop": stop}
