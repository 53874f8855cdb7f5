"""Mixed-step benchmark on one MI355X: the 7B-like layer at token budget 512.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: 32 query / 32 KV heads, head dim 128, KV blocks of 16 tokens, bf16; 64 running decodes
with contexts uniform on [512, 4096] and one 4096-token prompt under a budget of 512 tokens per
step (64 decode rows + 448 chunk rows; the prompt's life is 10 steps: nine 448-token chunks and a
64-token one).  A step is one pass of the whole hot path over one batch: the host batch build
(C++), one host-to-device metadata copy, the rope + paged-KV-append kernel and the mixed
attention (decode stage split, one kernel of decode waves and chunk tiles, combine).  The benchmark cycles through the prompt's ten
steps, restoring the builder from a snapshot after each cycle (re-appending identical K/V to
identical slots leaves the cache unchanged).  Every step's raw q/k/v are generated and resident in
HBM before the timed region.

Prints one JSON line.  ``roofline`` reports the dominant kernel (the attention kernel, whose decode
waves stream the cache, bound by HBM): algorithmic bytes per launch (K and V of every decode
context and of every chunk's visible keys, plus q and out) divided by its average duration,
measured with HIP events on the launch stream over every launch of a dedicated pass of whole
cycles after the timed loop (at least 20 launches).  ``isolated`` times decode-only and
chunk-only launches of the same metadata, warm and with L2 and MALL evicted by a read-only sweep,
and beside them the same chunks through torch's attention library (a reference point).
``graph_replay`` times the same steps replayed from HIP graphs (one per step shape, and with
padded token buckets), on this workload, on a serving-like stream whose token count changes
every step, and on a scaled-down workload whose short device steps leave the host's launches
setting the step time.  ``cpu_baseline`` times the CPU oracle (reference builder + rotary embedding + fp64
full-prefill attention) on every step of the cycle: all decode rows and a fixed subset of each
step's chunk rows, extrapolated to whole steps.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mixed-step tokens/s + step latency; % bf16 MFMA peak (chunks), % HBM BW (decode)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload index (default: the budget-512 layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--no-graphs", action="store_true",
                    help="skip the HIP-graph legs (replays of the same steps, exact shapes and "
                         "padded buckets, on this workload and on the serving-like stream)")
    ap.add_argument("--cpu-chunk-rows", type=int, default=32,
                    help="chunk rows per step the CPU baseline computes")
    ap.add_argument("--cpu-decode-rows", type=int, default=16,
                    help="decode rows per step the CPU baseline computes")
    ap.add_argument("--only", choices=("chunk", "decode"), default=None,
                    help="after the warm-up, run only isolated launches of one kind (chunk-only or "
                         "decode-only launches of every step's metadata, --reps each), print their "
                         "summary and exit: a run whose attention dispatches are all of that kind, "
                         "for profiler counters")
    ap.add_argument("--reps", type=int, default=5, help="launches per step with --only")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB before timing (a known-size kernel "
                         "for scaling profiler byte counters)")
    return ap.parse_args()


def decode_bytes(meta, w, elt: int) -> int:
    """Algorithmic HBM bytes of the decode rows: K and V of every visible key, q and out."""
    nd = meta.num_decodes
    ctx = int(meta.host["context_lens"][:nd].sum())
    return ctx * w.Hkv * w.D * 2 * elt + 2 * nd * w.Hq * w.D * elt


def chunk_bytes(meta, w, elt: int) -> int:
    """Algorithmic HBM bytes of the chunk rows: K and V of each chunk's visible keys (its cached
    prefix and itself) once, q and out."""
    nd, ns = meta.num_decodes, meta.num_seqs
    ctx = int(meta.host["context_lens"][nd:ns].sum())
    rows = meta.num_tokens - nd
    return ctx * w.Hkv * w.D * 2 * elt + 2 * rows * w.Hq * w.D * elt


def chunk_flops(meta, w) -> int:
    """Algorithmic FLOPs of the chunk rows: 4 D Hq per visible (row, key) pair (QK^T and PV)."""
    nd = meta.num_decodes
    pos = meta.host["positions"][nd:meta.num_tokens].long()
    return int((pos + 1).sum()) * 4 * w.D * w.Hq


TRAFFIC_WORKLOAD = "cfg2_7b_b512_bf16"     # the workload the committed counter summary covers


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch of ``kernel`` from the committed counter summary, or None when the
    summary covers another workload or the attention source has changed since it was taken."""
    import hashlib
    if workload != TRAFFIC_WORKLOAD:
        return None
    path = os.path.join(ROOT, "profiles", "hbm_traffic_b512_7b_layer.json")
    src = os.path.join(ROOT, "chunked_prefill_mixed_decode_amd", "csrc", "attention.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None
    if rec.get("source_sha256_16") != h:
        return None
    return rec["kernels"][kernel]["traffic_bytes"]


def isolation_pass(g, metas, qrots, outs, w, reps: int, flush=None, kinds=("decode", "chunk")):
    """Decode-only and chunk-only launches of each step's metadata, timed with HIP events on the
    launch stream: per-kernel durations without the other kernel running beside it.  The launches
    of one kind run back to back after one untimed launch, so the device is busy when each starts
    (as in a serving loop; a launch onto an idle device starts its workgroups over ~2 µs more).
    Decode launches report attention + combine time.  With ``flush`` (a device tensor larger than
    L2 and the MALL together), a read-only sum over it runs on the same stream before every timed
    launch, so that the caches hold none of the step's data and no dirty lines (cold cache)."""
    import torch
    cb = g.cb
    dec, chk = [], []

    def events(n):
        evs = [[timing_event() for _ in range(n)] for _ in range(reps)]
        for row in evs:
            for e in row:
                e.record()                       # touched once before the timed launches
        return evs

    for k, meta in enumerate(metas):
        nd, T = meta.num_decodes, meta.num_tokens
        h = meta.host
        dev = {kk: vv.to(g.device) for kk, vv in h.items()}
        cu_chunk = (dev["cu_seqlens_q"][nd:] - nd).contiguous()
        # Each launch shape plans its own split (a chunk-only launch splits keys further).
        Hq, Hkv, D = g.runner.Hq, g.runner.Hkv, g.runner.D
        need = [cb.cb_attn_workspace_bytes(nd, nd, nd, 1, meta.max_decode_context_len,
                                           meta.max_decode_context_len, Hq, Hkv, D)]
        # A chunk-only launch sizes its key split by its own rows' longest context.
        chunk_ctx = int(h["context_lens"][nd:meta.num_seqs].max()) if T > nd else 0
        need_chunk = 0
        if T > nd:
            need_chunk = cb.cb_attn_workspace_bytes(meta.num_seqs - nd, 0, T - nd, meta.max_q_len, 0,
                                                    chunk_ctx, Hq, Hkv, D)
            need.append(need_chunk)
        g.runner.ensure_workspace(max(need))

        def decode_launch(evs):
            cb.cb_mixed_paged_attention(
                qrots[k][:nd], g.runner.k_cache, g.runner.v_cache, dev["cu_seqlens_q"],
                dev["context_lens"], dev["cu_blocks"], dev["block_table"], outs[k][:nd],
                g.runner.workspace, num_seqs=nd, num_decodes=nd, max_q_len=1,
                max_decode_ctx=meta.max_decode_context_len, max_ctx=meta.max_decode_context_len,
                scale=g.runner.scale, events=evs)

        def chunk_launch(evs):
            cb.cb_mixed_paged_attention(
                qrots[k][nd:], g.runner.k_cache, g.runner.v_cache, cu_chunk,
                dev["context_lens"][nd:], dev["cu_blocks"][nd:], dev["block_table"], outs[k][nd:],
                g.runner.workspace, num_seqs=meta.num_seqs - nd, num_decodes=0,
                max_q_len=meta.max_q_len, max_decode_ctx=0, max_ctx=chunk_ctx,
                scale=g.runner.scale, events=evs)

        if nd > 0 and "decode" in kinds:
            ev = events(4)
            torch.cuda.synchronize()
            decode_launch(None)
            for r in range(reps):
                if flush is not None:
                    flush.sum()
                decode_launch([ev[r][0], ev[r][1], None, None, ev[r][2], ev[r][3]])
            torch.cuda.synchronize()
            for r in range(reps):
                dec.append((k, ev[r][0].elapsed_time(ev[r][1]) + ev[r][2].elapsed_time(ev[r][3])))
        if T > nd and "chunk" in kinds:
            # Timed twice: from the attention kernel's start to the combine's end (the launch splits
            # keys, and so has a combine, exactly when it needs a workspace), and around the
            # attention kernel alone.
            end_slot = 5 if need_chunk > 0 else 3
            whole, alone = events(2), events(2)
            torch.cuda.synchronize()
            chunk_launch(None)
            for evl, (s0, s1) in ((whole, (2, end_slot)), (alone, (2, 3))):
                for r in range(reps):
                    if flush is not None:
                        flush.sum()
                    evs6 = [None] * 6
                    evs6[s0], evs6[s1] = evl[r]
                    chunk_launch(evs6)
            torch.cuda.synchronize()
            for r in range(reps):
                chk.append((k, whole[r][0].elapsed_time(whole[r][1]), alone[r][0].elapsed_time(alone[r][1])))
    return dec, chk


def timing_event():
    """A HIP timing event recorded without the system-scope fence (``runner.HipEvent``): a default
    event's record writes back the device's caches before it completes, time that lands inside the
    interval it brackets."""
    from chunked_prefill_mixed_decode_amd.runner import HipEvent
    return HipEvent(timing=True)


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def linear_pass(w, dev, tokens: dict, reps: int = 20):
    """The linear layers around the step (selective batching: one weight read serves every token of
    the step): the QKV projection [T, Hq D] -> [T, (Hq + 2 Hkv) D] and the output projection
    [T, Hq D] -> [T, Hq D], with seeded synthetic weights, timed with HIP events on the launch
    stream at the decode-only and the mixed step's token counts.  Beside each, the same product
    through torch.matmul (the ROCm GEMM libraries; a reference point, never the product path)."""
    import torch
    from chunked_prefill_mixed_decode_amd import binding as cb
    from synth.values import matrix_values
    d = w.Hq * w.D
    layers = {"qkv_projection": (d, (w.Hq + 2 * w.Hkv) * w.D, "w_qkv"), "output_projection": (d, d, "w_o")}
    res = {}
    for lname, (K, N, wname) in layers.items():
        wt = matrix_values(7, wname, N, K, scale=K ** -0.5, dtype=torch.bfloat16, device=dev)
        for tname, T in tokens.items():
            x = matrix_values(7, "hidden", T, K, dtype=torch.bfloat16, device=dev)
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            nws = cb.cb_linear_workspace_bytes(T, N, K)
            ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
            cb.cb_linear(x, wt, y, ws)
            e0, e1 = timing_event(), timing_event()
            e0.record()
            for _ in range(reps):
                cb.cb_linear(x, wt, y, ws)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            flop = 2 * T * K * N
            wbytes = K * N * 2
            wT = wt.t().contiguous()                  # [K, N]: the library's plain row-major operand
            torch.matmul(x, wT)
            e0.record()
            for _ in range(reps):
                torch.matmul(x, wT)
            e1.record()
            torch.cuda.synchronize()
            lib_us = e0.elapsed_time(e1) / reps * 1e3
            del wT
            res[f"{lname}_{tname}"] = {
                "tokens": T, "K": K, "N": N, "us": us, "TFLOPs": flop / us / 1e6,
                "frac_mfma": flop / us / 1e6 / MFMA_BF16_PEAK_TFLOPS,
                "library_matmul_us": lib_us, "library_frac_mfma": flop / lib_us / 1e6 / MFMA_BF16_PEAK_TFLOPS,
                "weight_GBps": wbytes / us / 1e3,
                "flop_per_weight_byte": flop / wbytes, "k_splits": nws // (T * N * 4) if nws else 1}
            del x, y, ws
        del wt
    return res


def summarize_isolated(dec, chk, metas, w, elt):
    """Roofline fractions of isolated launches: decode rows (bytes over attention + combine time)
    against HBM, chunk rows (FLOPs over attention + combine time when the launch splits keys; the
    attention kernel alone beside it) against bf16 MFMA, totals and per step."""
    dec_s = sum(t for _, t in dec) / 1e3
    chk_s = sum(t for _, t, _ in chk) / 1e3
    chk_attn_s = sum(t for _, _, t in chk) / 1e3
    dbytes = sum(decode_bytes(metas[k], w, elt) for k, _ in dec)
    cflops = sum(chunk_flops(metas[k], w) for k, _, _ in chk)
    per_step = {}
    for k, t, _ in chk:
        per_step.setdefault(k, []).append(t)
    out = {"decode_avg_us": dec_s / max(1, len(dec)) * 1e6,
           "decode_GBps": dbytes / max(dec_s, 1e-12) / 1e9,
           "decode_frac_hbm": dbytes / max(dec_s, 1e-12) / 1e9 / HBM_PEAK_GBS,
           "chunk_avg_us": chk_s / max(1, len(chk)) * 1e6,
           "chunk_TFLOPs": cflops / max(chk_s, 1e-12) / 1e12,
           "chunk_frac_mfma": cflops / max(chk_s, 1e-12) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "chunk_attn_kernel_avg_us": chk_attn_s / max(1, len(chk)) * 1e6,
           "chunk_attn_kernel_frac_mfma": cflops / max(chk_attn_s, 1e-12) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "chunk_flops_per_step": cflops / max(1, len(chk)),
           "chunk_TFLOPs_per_step": {str(k): chunk_flops(metas[k], w) / (sum(v) / len(v) / 1e3) / 1e12
                                     for k, v in sorted(per_step.items())}}
    return out


def library_attention(metas, w, dev, reps: int = 3, max_keys: int = 65536):
    """The chunk rows of each step through torch's scaled_dot_product_attention (the ROCm
    attention libraries; a reference point, never the product path): per chunk, contiguous
    [1, H, len, D] query, key and value tensors of random bf16 values with a bottom-right causal
    mask (row i of a chunk after c cached keys sees keys 0..c + i), timed with HIP events over
    ``reps`` calls per step after one untimed call.  The library reads contiguous keys, not the
    paged cache.  None when a chunk sees more than ``max_keys`` keys."""
    import torch
    from torch.nn.attention.bias import causal_lower_right
    steps, flops = [], 0
    for k, meta in enumerate(metas):
        nd, S = meta.num_decodes, meta.num_seqs
        cu = meta.host["cu_seqlens_q"]
        ctx = meta.host["context_lens"]
        shapes = [(int(cu[s + 1] - cu[s]), int(ctx[s])) for s in range(nd, S)]
        if not shapes:
            continue
        if max(c for _, c in shapes) > max_keys:
            return None
        ts = []
        for d, c in shapes:
            q = torch.randn(1, w.Hq, d, w.D, dtype=torch.bfloat16, device=dev)
            kv = [torch.randn(1, w.Hkv, c, w.D, dtype=torch.bfloat16, device=dev) for _ in range(2)]
            mask = causal_lower_right(d, c)

            def call():
                return torch.nn.functional.scaled_dot_product_attention(q, kv[0], kv[1], attn_mask=mask,
                                                                        enable_gqa=w.Hq != w.Hkv)
            call()
            e0, e1 = timing_event(), timing_event()
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / reps * 1e3)
        steps.append(sum(ts))
        flops += chunk_flops(meta, w)
    if not steps:
        return None
    tot = sum(steps)
    return {"us_per_step": tot / len(steps), "TFLOPs": flops / tot / 1e6,
            "frac_mfma": flops / tot / 1e6 / MFMA_BF16_PEAK_TFLOPS,
            "note": "torch scaled_dot_product_attention on each step's chunks (contiguous K/V, bottom-right "
                    "causal mask, random bf16 values); a library reference point beside chunk_frac_mfma"}


def cpu_baseline(w, n_steps: int, chunk_rows: int, decode_rows: int):
    """The oracle on every step of the cycle, in order: the Python reference builder, then for a
    fixed subset of each step's rows (``decode_rows`` of the decode rows and ``chunk_rows`` of the
    chunk rows: the first and last quarter of each kind, the rest seeded random) the rotary
    embedding of the row's sequence's keys and of its query, and fp64 attention.  Each part is
    timed; a step's oracle time is extrapolated to all of its rows (decode sequences by count,
    chunk-row attention by rows; a chunk's keys are rotated in full either way).  Raw inputs are
    generated before each step's timed part."""
    import numpy as np

    from oracle import attention as oattn
    from oracle import rope as orope
    from oracle.builder import RefBuilder
    from synth import values
    from tests.gpu_harness import TORCH_DTYPE

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    b = RefBuilder(w.block_size, w.num_blocks, w.free_list)
    for c in w.decode_ctx:
        b.add_running(c)
    for L, cached in w.prompts:
        b.add_prompt(L, cached)
    dt = TORCH_DTYPE[w.dtype]
    table = orope.cos_sin_table(w.max_position(), w.D)
    scale = 1.0 / np.sqrt(w.D)
    rng = np.random.default_rng(0)

    def subset(rows, n):
        rows = np.asarray(rows)
        if len(rows) <= n:
            return set(rows.tolist())
        q = n // 4
        out = set(rows[:q].tolist()) | set(rows[-q:].tolist())
        return out | set(rng.choice(rows[q:-q], size=n - 2 * q, replace=False).tolist())

    per_step, rows_done, tokens, est = [], 0, 0, 0.0
    for step in range(n_steps):
        probe = b.clone().build(w.budget)
        nd, T = probe["num_decodes"], probe["num_tokens"]
        cu = probe["cu_seqlens_q"]
        pick = subset(range(nd), decode_rows) | subset(range(nd, T), chunk_rows)
        raw = {}
        for s in range(probe["num_seqs"]):
            rows = [r for r in range(cu[s], cu[s + 1]) if r in pick]
            if not rows:
                continue
            rid = probe["seq_ids"][s]
            pos = [probe["positions"][r] for r in rows]
            last = probe["context_lens"][s]
            raw[rid] = (values.range_values(w.seed, "k", rid, 0, last, w.Hkv, w.D, dt).float().numpy(),
                        values.range_values(w.seed, "v", rid, 0, last, w.Hkv, w.D, dt).float().numpy(),
                        values.token_values(w.seed, "q", rid, pos, w.Hq, w.D, dt).float().numpy(),
                        np.array(pos))
        t0 = time.perf_counter()
        plan = b.build(w.budget)
        t_build = time.perf_counter() - t0
        t_dec = t_chk_rot = t_chk_att = 0.0
        n_dec = n_chk = 0
        for s in range(plan["num_seqs"]):
            rid = plan["seq_ids"][s]
            if rid not in raw:
                continue
            k, v, q, pos = raw[rid]
            t1 = time.perf_counter()
            kh = orope.rotate_stored(k, np.arange(k.shape[0]), table, w.dtype)
            qh = orope.rotate_stored(q, pos, table, w.dtype)
            t2 = time.perf_counter()
            oattn.attend(qh, kh, v, pos, scale)
            t3 = time.perf_counter()
            if s < nd:
                t_dec += t3 - t1
                n_dec += 1
            else:
                t_chk_rot += t2 - t1
                t_chk_att += t3 - t2
                n_chk += len(pos)
        rows_done += n_dec + n_chk
        full = (t_build + (t_dec * nd / n_dec if n_dec else 0.0) + t_chk_rot +
                (t_chk_att * (T - nd) / n_chk if n_chk else 0.0))
        est += full
        tokens += T
        per_step.append({"step": step, "tokens": T, "rows_computed": n_dec + n_chk,
                         "seconds": t_build + t_dec + t_chk_rot + t_chk_att, "seconds_full_step": full})
        del raw
    measured = sum(p["seconds"] for p in per_step)
    return {"value": tokens / est, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "seconds": measured, "per_step": per_step,
            "sample": f"every step of the {n_steps}-step cycle: reference builder, then rotary embedding and "
                      f"fp64 causal attention of {decode_rows} decode rows and {chunk_rows} chunk rows per step "
                      f"(first and last quarter of each kind, the rest seeded random; {rows_done} rows x "
                      f"{w.Hq} heads in {measured:.1f} s); value = the cycle's tokens over the oracle time "
                      f"extrapolated to every row of every step ({est:.1f} s)"}


def graph_legs(g, w, snap, inputs, cycle: int, steps: int, arrivals: bool = False):
    """The cycle's steps eagerly, replayed from one HIP graph per step shape (runner.StepGraphs,
    captured on first occurrence), and replayed from one graph per padded shape (runner.Buckets:
    token count and longest query to a multiple of 64, longest contexts to a multiple of 4096,
    padding rows skipped by the append).  ``steps`` timed steps each; host wall time with a device
    sync on both sides.  Row buffers of a padded shape keep the inputs of the first step that used
    it (timing only)."""
    import torch

    from chunked_prefill_mixed_decode_amd.runner import Buckets, StepGraphs
    cb = g.cb
    r = g.runner
    bk = Buckets(tokens=64, context=4096)
    st = {"sched": cb.cb_sched_clone(snap), "k": 0}

    def restart():
        st["sched"], st["k"] = cb.cb_sched_clone(snap), 0

    def build(buckets=None):
        k = st["k"]
        if arrivals:
            g.arrive(k, st["sched"])
        return k, r.build(st["sched"], w.budget, buckets=buckets)

    def advance():
        st["k"] += 1
        if st["k"] == cycle:
            restart()

    # Workspace for every exact and padded shape of the cycle (a reallocation drops the graphs).
    need = 0
    for buckets in (None, bk):
        restart()
        for _ in range(cycle):
            _, meta = build(buckets)
            need = max(need, r.workspace_bytes(meta))
            advance()
    r.ensure_workspace(need)
    q_rot = [torch.empty_like(x[0]) for x in inputs]
    out = [torch.empty_like(x[0]) for x in inputs]

    def timed(step_fn):
        restart()
        for _ in range(2 * cycle):             # warm-up; captures every shape (both pinned buffers)
            step_fn(False)
        torch.cuda.synchronize()
        restart()
        tok = 0
        t1 = time.perf_counter()
        for _ in range(steps):
            tok += step_fn(True)
        torch.cuda.synchronize()
        return tok, time.perf_counter() - t1

    def eager(count):
        k, meta = build()
        dm = r.upload(meta)
        q, kk, vv = inputs[k]
        r.append(dm, q, kk, vv, q_rot[k])
        r.attend(meta, dm, q_rot[k], out[k])
        advance()
        return meta.num_tokens

    graphs, modes = StepGraphs(r), set()

    def replay(count):
        k, meta = build()
        q, kk, vv = inputs[k]

        def launch(dm):
            r.append(dm, q, kk, vv, q_rot[k])
            r.attend(meta, dm, q_rot[k], out[k])
        m = graphs.step(meta, launch)
        if count:
            modes.add(m)
        advance()
        return meta.num_tokens

    bgraphs, bmodes, rows, pad = StepGraphs(r), set(), {}, {"rows": 0, "real": 0}

    def bucketed(count):
        k, meta = build(bk)
        key = StepGraphs.key(meta)
        if key not in rows:
            T, Tp = meta.num_tokens, meta.launch_tokens
            rows[key] = [torch.cat([x, x.new_zeros((Tp - T,) + x.shape[1:])]) for x in inputs[k]]
            rows[key] += [torch.empty_like(rows[key][0]), torch.empty_like(rows[key][0])]
        q, kk, vv, qr, o = rows[key]

        def launch(dm):
            r.append(dm, q, kk, vv, qr)
            r.attend(meta, dm, qr, o)
        m = bgraphs.step(meta, launch)
        if count:
            bmodes.add(m)
            pad["rows"] += meta.launch_tokens
            pad["real"] += meta.num_tokens
        advance()
        return meta.num_tokens

    etok, eel = timed(eager)
    gtok, gel = timed(replay)
    btok, bel = timed(bucketed)
    restart()
    return {
        "workload": w.name, "steps": steps, "cycle": cycle,
        "eager_ms_per_step": eel / steps * 1e3, "eager_tokens_per_s": etok / eel,
        "ms_per_step": gel / steps * 1e3, "value": gtok / gel, "unit": "tokens/s",
        "graphs": len(graphs.graphs), "all_replayed": modes == {"replay"},
        "bucketed": {"ms_per_step": bel / steps * 1e3, "value": btok / bel, "unit": "tokens/s",
                     "graphs": len(bgraphs.graphs), "all_replayed": bmodes == {"replay"},
                     "token_bucket": bk.tokens, "context_bucket": bk.context,
                     "padded_rows_frac": pad["rows"] / max(1, pad["real"]) - 1.0,
                     "us_saved_per_step_vs_eager": (eel - bel) / steps * 1e6},
        "us_saved_per_step_vs_eager": (eel - gel) / steps * 1e6,
        "note": "the cycle's steps eager, replayed from one HIP graph per exact step shape (and pinned "
                "buffer), and from one graph per padded shape; host wall time per step"}


def stream_graph_leg(dev, steps: int):
    """graph_legs on the serving-like stream (synth.workloads.stream_b512): the budget-512 layer's
    geometry with 64 decodes and prompts arriving over a 48-step cycle, so the token count (64 to
    512) and the decode count change from step to step and padding really occurs."""
    from synth import workloads
    from tests.gpu_harness import DeviceRun
    w = workloads.stream_b512()
    g = DeviceRun(w, dev, sentinel=False)
    cb = g.cb
    snap = cb.cb_sched_clone(g.sched)
    probe = cb.cb_sched_clone(snap)
    bufs = cb.StepBuffers(*g.runner.bufs[0].cap)
    inputs = []
    for k in range(w.steps):
        g.arrive(k, probe)
        meta = cb.cb_build_step(probe, w.budget, bufs)
        inputs.append(g.step_inputs(meta))
    res = graph_legs(g, w, snap, inputs, w.steps, max(steps, 2 * w.steps), arrivals=True)
    res["tokens_per_step_range"] = [min(x[0].shape[0] for x in inputs), max(x[0].shape[0] for x in inputs)]
    return res


def launch_bound_graph_leg(dev, steps: int):
    """graph_legs on a scaled-down workload whose device step (tens of microseconds) is shorter
    than the host's build and launches (5 query heads, 4 decodes at 300 cached tokens and a
    600-token prompt in 128-token chunks, a 6-step cycle): there the host's launch cost sets the
    step time, the regime in which replaying a captured step saves time."""
    from synth import workloads
    from tests.gpu_harness import DeviceRun
    w = workloads.small(3)
    g = DeviceRun(w, dev, sentinel=False)
    cb = g.cb
    snap = cb.cb_sched_clone(g.sched)
    probe = cb.cb_sched_clone(snap)
    bufs = cb.StepBuffers(*g.runner.bufs[0].cap)
    inputs = []
    for _ in range(w.steps):
        meta = cb.cb_build_step(probe, w.budget, bufs)
        inputs.append(g.step_inputs(meta))
    res = graph_legs(g, w, snap, inputs, w.steps, steps)
    res["tokens_per_step_range"] = [min(x[0].shape[0] for x in inputs), max(x[0].shape[0] for x in inputs)]
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path has no multi-GPU leg (--gpus {args.gpus} is not "
              f"supported; sharding is a design only)", file=sys.stderr)
        sys.exit(2)
    import torch

    from synth import workloads
    from tests.gpu_harness import DeviceRun

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = workloads.get(args.config)
    cb_steps = w.steps
    print(f"[bench] set-up {w.name}: {len(w.decode_ctx)} decodes, {w.num_blocks} blocks", file=sys.stderr, flush=True)
    g = DeviceRun(w, dev, sentinel=False)
    cb = g.cb
    snapshot = cb.cb_sched_clone(g.sched)

    # One dry cycle learns each step's metadata; its inputs are generated and kept in HBM.  A
    # workload without a fixed step count cycles until its last prompt has had its last chunk.
    if cb_steps is None:
        p2 = cb.cb_sched_clone(snapshot)
        b2 = cb.StepBuffers(*g.runner.bufs[0].cap)
        cb_steps = 0
        while cb.cb_sched_pending_prompts(p2) > 0 and cb_steps < w.max_steps:
            cb.cb_build_step(p2, w.budget, b2)
            cb_steps += 1
    inputs, metas, ws = [], [], 0
    probe = cb.cb_sched_clone(snapshot)
    bufs = cb.StepBuffers(*g.runner.bufs[0].cap)
    for k in range(cb_steps):
        meta = cb.cb_build_step(probe, w.budget, bufs)
        meta.host = {kk: vv.clone() for kk, vv in meta.host.items()}
        metas.append(meta)
        inputs.append(g.step_inputs(meta))
        ws = max(ws, g.runner.workspace_bytes(meta))
    g.runner.ensure_workspace(ws)
    outs = [torch.empty_like(inp[0]) for inp in inputs]
    qrots = [torch.empty_like(inp[0]) for inp in inputs]
    torch.cuda.synchronize()

    state = {"sched": cb.cb_sched_clone(snapshot), "k": 0}

    def one_step(events=None, bracket=None):
        k = state["k"]
        meta = g.runner.build(state["sched"], w.budget)
        if bracket is not None:
            bracket[0].record()
        dev_meta = g.runner.upload(meta)
        q, kk, vv = inputs[k]
        g.runner.append(dev_meta, q, kk, vv, qrots[k])
        g.runner.attend(meta, dev_meta, qrots[k], outs[k], events=events)
        if bracket is not None:
            bracket[1].record()
        state["k"] = k + 1
        if state["k"] == cb_steps:
            state["k"] = 0
            state["sched"] = cb.cb_sched_clone(snapshot)
        return meta.num_tokens, k

    if args.calib_copy_mib:
        # One device-to-device hipMemcpyAsync (the runtime's copy kernel) of a known size.
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        nbytes = args.calib_copy_mib << 20
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        rc = hip.hipMemcpyAsync(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                ctypes.c_size_t(nbytes), ctypes.c_int(3),   # hipMemcpyDeviceToDevice
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync failed: {rc}")
        torch.cuda.synchronize()
        del src, dst
    # The step loop is host-driven: a collector pass over the set-up objects (tens of thousands:
    # tensors, metadata, the workload) stalls the host for about a millisecond every few steps,
    # long enough to drain the two steps queued ahead of the GPU.  Freezing them leaves the
    # collector only the few objects each step creates.
    gc.collect()
    gc.freeze()
    for _ in range(max(args.warmup, cb_steps if args.only else 0)):
        one_step()
    torch.cuda.synchronize()
    if args.only:
        print(f"[bench] {args.only}-only launches, {args.reps} per step...", file=sys.stderr, flush=True)
        dec_raw, chk_raw = isolation_pass(g, metas, qrots, outs, w, reps=args.reps, kinds=(args.only,))
        res = summarize_isolated(dec_raw, chk_raw, metas, w, 2)
        res.update({"only": args.only, "reps": args.reps, "workload": w.name})
        print(json.dumps(res), flush=True)
        return

    # The timed loop records no events: each record costs the GPU time of its own.
    tokens = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        n, _ = one_step()
        tokens += n
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    elt = 2

    # Event pass: whole cycles (at least 20 steps) with HIP events around every attention launch,
    # its combine and the whole step, after the timed loop: the roofline figure and the device
    # step latency (which therefore carries the records' own cost, a few µs a step).
    n_ev = cb_steps * max(2, -(-20 // cb_steps))
    ev_pass = [[timing_event() for _ in range(8)] for _ in range(n_ev)]
    for e8 in ev_pass:
        for e in e8:
            e.record()
    torch.cuda.synchronize()
    state["sched"], state["k"] = cb.cb_sched_clone(snapshot), 0
    ev_steps = []
    for e8 in ev_pass:
        _, k = one_step(e8[:6], e8[6:])
        ev_steps.append(k)
    torch.cuda.synchronize()
    dec_ms = [e8[0].elapsed_time(e8[1]) for e8 in ev_pass]      # the attention kernel
    dev_step_ms = [e8[6].elapsed_time(e8[7]) for e8 in ev_pass]
    cmb_ms = [e8[4].elapsed_time(e8[5]) for e8 in ev_pass]
    abytes = [decode_bytes(metas[k], w, elt) + chunk_bytes(metas[k], w, elt) for k in ev_steps]
    attn_avg_s = sum(dec_ms) / len(dec_ms) / 1e3
    achieved = sum(abytes) / len(abytes) / attn_avg_s / 1e9
    state["sched"], state["k"] = cb.cb_sched_clone(snapshot), 0

    graph_rep = None
    if not args.no_graphs:
        print("[bench] graph replay legs...", file=sys.stderr, flush=True)
        graph_rep = graph_legs(g, w, snapshot, inputs, cb_steps, args.steps)
        graph_rep["varying"] = stream_graph_leg(dev, args.steps)
        graph_rep["launch_bound"] = launch_bound_graph_leg(dev, args.steps)
        state["sched"], state["k"] = cb.cb_sched_clone(snapshot), 0

    # End-to-end latency: host wall time from cb_build_step to stream sync after attention.
    e2e = []
    for _ in range(min(args.steps, 3 * cb_steps)):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        one_step()
        torch.cuda.synchronize()
        e2e.append((time.perf_counter() - t1) * 1e3)

    print("[bench] isolated launches (warm, then cold)...", file=sys.stderr, flush=True)
    dec_raw, chk_raw = isolation_pass(g, metas, qrots, outs, w, reps=3)
    iso = summarize_isolated(dec_raw, chk_raw, metas, w, elt)
    iso["note"] = ("decode-only and chunk-only launches of the same step metadata, 3 timed per step and kind, "
                   "back to back after one untimed launch")
    iso["library_chunk_attention"] = library_attention(metas, w, dev)
    flush = torch.ones(256 << 20, dtype=torch.int32, device=dev)    # 1 GiB, written once here
    torch.cuda.synchronize()
    iso_cold = summarize_isolated(*isolation_pass(g, metas, qrots, outs, w, reps=2, flush=flush), metas, w, elt)
    iso_cold["note"] = ("as isolated, with a read-only sweep of 1 GiB on the stream before every timed "
                        "launch (L2 and MALL hold none of the step's data and no dirty lines)")
    del flush
    traffic = committed_traffic("attn_kernel", w.name)
    # What the chunk rows add to a mixed step: the in-step attention + combine minus the warm
    # decode-only launch of the same step's metadata, per event-pass step with chunk rows.
    iso_dec = {}
    for k, t in dec_raw:
        iso_dec.setdefault(k, []).append(t)
    marg, mflops = [], []
    for e8, k in zip(ev_pass, ev_steps):
        if k in iso_dec and chunk_flops(metas[k], w) > 0:
            marg.append(e8[0].elapsed_time(e8[1]) + e8[4].elapsed_time(e8[5]) - sum(iso_dec[k]) / len(iso_dec[k]))
            mflops.append(chunk_flops(metas[k], w))
    chunk_marginal = None
    if marg:
        m_s = sum(marg) / len(marg) / 1e3
        f = sum(mflops) / len(mflops)
        iso_chk = {}
        for k, t, _ in chk_raw:
            iso_chk.setdefault(k, []).append(t)
        alone = [sum(iso_chk[k]) / len(iso_chk[k]) for k in ev_steps if k in iso_chk and k in iso_dec]
        alone_us = sum(alone) / len(alone) * 1e3 if alone else None
        chunk_marginal = {"us_per_step": m_s * 1e6, "chunk_flops_per_step": f,
                          "chunk_only_us": alone_us,
                          "hidden_frac": (1.0 - m_s * 1e6 / alone_us) if alone_us else None,
                          "steps": len(marg),
                          "note": "time the chunk rows add to the mixed step (in-step attention + combine "
                                  "minus the warm decode-only launch of the same metadata) against the "
                                  "chunk-only launch of the same steps: the share of the chunk work hidden "
                                  "under the decode rows' streaming; a step cost, not a utilisation"}
    lin = linear_pass(w, dev, {"decode_only": max(1, len(w.decode_ctx)),
                               "mixed_step": max(m.num_tokens for m in metas)}) if w.dtype == "bf16" else None

    res = {
        "metric": METRIC,
        "value": tokens / el,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": el / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded SplitMix64 normal-quantile activations; seeded workload structure)",
        "config": {"workload": w.name, "heads_q": w.Hq, "heads_kv": w.Hkv, "head_dim": w.D,
                   "block_size": w.block_size, "token_budget": w.budget,
                   "decodes": len(w.decode_ctx), "prompts": [list(p) for p in w.prompts],
                   "steps_per_cycle": cb_steps, "parallelism": "1 GPU"},
        "roofline": {"bound": "hbm", "kernel": "attn_kernel (decode waves + chunk tiles, one launch)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "bytes_per_launch": sum(abytes) / len(abytes), "avg_launch_us": attn_avg_s * 1e6,
                     "launches_timed": len(dec_ms)},
        "isolated": iso,
        "isolated_cold": iso_cold,
        "chunk_marginal": chunk_marginal,
        "linear_layers": lin,
        "combine_avg_us": sum(cmb_ms) / len(cmb_ms) * 1e3,
        "device_step_us": sum(dev_step_ms) / len(dev_step_ms) * 1e3,
        "device_step_us_p10_p50_p90": [pct(dev_step_ms, q) * 1e3 for q in (0.1, 0.5, 0.9)],
        "end_to_end_ms_p10_p50_p90": [pct(e2e, q) for q in (0.1, 0.5, 0.9)],
        "event_pass_steps": len(dec_ms),
        "graph_replay": graph_rep,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, cb_steps, args.cpu_chunk_rows, args.cpu_decode_rows)
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
