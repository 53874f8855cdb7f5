"""Step-level simulation of the batch builder under a request stream.

Each step admits the requests that arrive at it (``cb_sched_add_prompt``), builds the step
(``cb_build_step``) and books the tokens it produces: the step that runs a prompt's last chunk
produces that request's first token ("Chunked Prefill 的 Token 预算" §03: a prompt whose prefill
completes turns into a decode), every decode row one more.  A request that has produced all its
output tokens is retired (``cb_sched_finish``) and its blocks return to the pool.  Reported, in
steps: time to first token (first-token step - arrival + 1) and time between tokens (steps between
consecutive tokens of one request), the two metrics "Splitting Prefill From Decode Inside a Step"
weighs the priority orders by ("Choosing the priority order") and "Chunked Prefill 的 Token 预算"
§08-§09 trade against each other.  No GPU work: the builder is the product's C++ one.

    python -m chunked_prefill_mixed_decode_amd.sim      # policy comparison on a seeded stream
"""
from __future__ import annotations

import argparse
import dataclasses
import json

from . import binding as cb


@dataclasses.dataclass
class SimResult:
    steps: int                       # steps simulated
    ttft: dict                       # request index -> steps from arrival to first token
    tbt: list                        # every gap (in steps) between consecutive tokens of a request
    finished: int                    # requests that produced all their tokens
    tokens: int                      # query tokens scheduled over the run
    unused: int                      # budget tokens left unused over the run
    stop: str                        # "" or the builder error that ended the run


def simulate(stream, budget: int, steps: int, *, running=(), block_size: int = 16,
             num_blocks: int = 1 << 16, cap_seqs: int = 4096, **cfg) -> SimResult:
    """Run up to ``steps`` steps (fewer once every request is done) of the builder (configured by ``cfg``: cb_sched_create's caps and
    policy) over ``stream`` (synth.streams.Request items, by arrival).  ``running`` lists
    (context_len, output_len) of requests already decoding when step 1 starts; in the results they
    follow the stream's requests (index len(stream) + j)."""
    s = cb.cb_sched_create(block_size, num_blocks, **cfg)
    buf = cb.StepBuffers(cap_seqs, budget, num_blocks, pin=False)
    req_of, done, produced, last_tok = {}, {}, {}, {}
    outputs = [r.output_len for r in stream] + [o for _, o in running]
    for j, (ctx, _) in enumerate(running):
        rid = cb.cb_sched_add_running(s, ctx)
        req_of[rid], produced[rid], last_tok[rid] = len(stream) + j, 0, 0
    ttft, tbt = {}, []
    tokens = unused = finished = 0
    stop = ""
    nxt = 0
    t = 0
    for t in range(1, steps + 1):
        while nxt < len(stream) and stream[nxt].arrival <= t:
            r = stream[nxt]
            rid = cb.cb_sched_add_prompt(s, r.prompt_len, r.cached_len)
            req_of[rid], done[rid], produced[rid] = nxt, r.cached_len, 0
            nxt += 1
        try:
            m = cb.cb_build_step(s, budget, buf)
        except cb.CbError as e:
            stop = cb._lib().cb_status_string(e.status).decode()
            break
        tokens += m.num_tokens
        unused += m.unused_tokens
        ids = m.host["seq_ids"].tolist()
        cu = m.host["cu_seqlens_q"].tolist()
        out_now = []
        for k, rid in enumerate(ids):
            i = req_of[rid]
            if k >= m.num_decodes:                       # a chunk: the prompt's end gives token 1
                done[rid] += cu[k + 1] - cu[k]
                if done[rid] < stream[i].prompt_len:
                    continue
                ttft[i] = t - stream[i].arrival + 1
            else:
                tbt.append(t - last_tok[rid])
            produced[rid] += 1
            last_tok[rid] = t
            if produced[rid] == outputs[i]:
                out_now.append(rid)
        for rid in out_now:
            cb.cb_sched_finish(s, rid)
            finished += 1
        if nxt == len(stream) and finished == len(outputs):
            break                                        # every request is done
    return SimResult(t, ttft, tbt, finished, tokens, unused, stop)


def _pct(xs, q):
    if not xs:
        return None
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(q * len(xs)))]


def summarize(res: SimResult, n_requests: int, budget: int) -> dict:
    tt = list(res.ttft.values())
    return {"steps": res.steps, "first_tokens": len(tt), "requests": n_requests,
            "finished": res.finished, "stop": res.stop,
            "ttft_p50": _pct(tt, 0.5), "ttft_p90": _pct(tt, 0.9), "ttft_p99": _pct(tt, 0.99),
            "ttft_max": max(tt, default=None),
            "tbt_mean": round(sum(res.tbt) / len(res.tbt), 3) if res.tbt else None,
            "tbt_p99": _pct(res.tbt, 0.99), "tbt_max": max(res.tbt, default=None),
            "budget_used": round(res.tokens / (res.tokens + res.unused), 4) if res.tokens + res.unused else None}


POLICIES = {
    "decode-first": {},
    "decode-first + 25% prefill quota": {"prefill_quota_pct": 25},
    "prefill-first": {"policy": cb.CB_POLICY_PREFILL_FIRST},
    "fair share 50/50": {"policy": cb.CB_POLICY_FAIR_SHARE, "decode_share_pct": 50},
    "decode-first, threshold ceiling 512": {"max_chunk": 512},
    "decode-first, floor 512": {"prefill_floor": 512},
}


def main():
    from synth.streams import mixed_stream
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--requests", type=int, default=300)
    ap.add_argument("--steps", type=int, default=3000)
    a = ap.parse_args()
    # Mixed traffic: log-normal prompts (median 1500) every ~1.2 steps, budget 2048.
    mixed = mixed_stream(a.seed, a.requests, mean_gap=1.2)
    # Decode-heavy traffic ("Chunked Prefill 的 Token 预算" §08): 240 decodes that outlive the run
    # hold most of a 256-token budget while prompts of median 300 arrive every ~4 steps.
    heavy = mixed_stream(a.seed + 1, a.requests // 4, mean_gap=4.0, median_prompt=300, sigma=0.5)
    scenarios = [("mixed, budget 2048", mixed, 2048, ()),
                 ("decode-heavy, budget 256", heavy, 256, [(1000, 10 ** 9)] * 240)]
    for label, stream, budget, running in scenarios:
        for name, cfg in POLICIES.items():
            res = simulate(stream, budget, a.steps, running=running, **cfg)
            print(json.dumps({"traffic": label, "policy": name, **summarize(res, len(stream), budget)}),
                  flush=True)


if __name__ == "__main__":
    main()
