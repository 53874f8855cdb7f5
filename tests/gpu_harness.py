"""GPU-side set-up of a workload: the HIP path through the binding, with seeded inputs from
``synth``.  Imports nothing from ``oracle/`` (the benchmark uses it outside its CPU-baseline leg).
"""
from __future__ import annotations

import numpy as np
import torch

from synth import values, workloads

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def cached_tokens(w: workloads.Workload):
    """(request id, tokens already in the cache) for every request at set-up."""
    out = [(i, c) for i, c in enumerate(w.decode_ctx)]
    nd = len(w.decode_ctx)
    out += [(nd + j, cached) for j, (_, cached) in enumerate(w.prompts) if cached > 0]
    return out


def step_caps(w: workloads.Workload, budget: int | None = None):
    """Capacities for one step's metadata arrays (for budgets up to ``budget``)."""
    prompts = list(w.prompts) + [(L, c) for _, L, c in w.arrivals]
    n_req = len(w.decode_ctx) + len(prompts)
    tokens = max(w.budget, budget or 0)
    blocks = sum(-(-(c + (w.steps or w.max_steps) + 1) // w.block_size) for c in w.decode_ctx)
    blocks += sum(-(-(L + (w.steps or w.max_steps) + 1) // w.block_size) for L, _ in prompts)
    return n_req, tokens, blocks


# ---------------------------------------------------------------------------------------------
# HIP side
# ---------------------------------------------------------------------------------------------
class DeviceRun:
    def __init__(self, w: workloads.Workload, device="cuda", sentinel=True, populate=True,
                 max_budget: int | None = None, sched_cfg: dict | None = None):
        from chunked_prefill_mixed_decode_amd import binding as cb
        from chunked_prefill_mixed_decode_amd.runner import MixedStepRunner
        self.cb = cb
        self.w = w
        self.device = torch.device(device)
        self.dtype = TORCH_DTYPE[w.dtype]
        self.sched = cb.cb_sched_create(w.block_size, w.num_blocks, w.free_list, **(sched_cfg or {}))
        for c in w.decode_ctx:
            cb.cb_sched_add_running(self.sched, c)
        for L, cached in w.prompts:
            cb.cb_sched_add_prompt(self.sched, L, cached)
        ns, nt, nb = step_caps(w, max_budget)
        self.runner = MixedStepRunner(Hq=w.Hq, Hkv=w.Hkv, D=w.D, block_size=w.block_size,
                                      num_blocks=w.num_blocks, dtype=self.dtype, device=self.device,
                                      max_pos=w.max_position(), cap_seqs=ns, cap_tokens=nt,
                                      cap_blocks=nb, sentinel=sentinel)
        self.written = 0                       # slots written so far
        self.step_index = 0                    # steps run by step()
        if populate:
            self.populate()

    def arrive(self, step: int, sched=None):
        """Queue the prompts that arrive before ``step``'s build (into ``sched``, default this run's)
        and write the K/V of their cached prefixes."""
        sched = self.sched if sched is None else sched
        for L, cached in self.w.arriving(step):
            rid = self.cb.cb_sched_add_prompt(sched, L, cached)
            if cached:
                self._write_cached(rid, cached, sched)

    def _write_cached(self, rid: int, n: int, sched):
        w, bs = self.w, self.w.block_size
        blocks = torch.tensor(self.cb.cb_sched_get_blocks(sched, rid), dtype=torch.int64, device=self.device)
        pos = torch.arange(n, dtype=torch.int64, device=self.device)
        slots = (blocks[pos // bs] * bs + pos % bs).to(torch.int32)
        k = values.token_values(w.seed, "k", rid, pos, w.Hkv, w.D, self.dtype, self.device)
        v = values.token_values(w.seed, "v", rid, pos, w.Hkv, w.D, self.dtype, self.device)
        self.runner.append_rows(pos.to(torch.int32), slots, k, v)
        self.written += n

    def populate(self, rows_per_batch: int = 1 << 16):
        """Write K/V of every token that is already cached at set-up into its slots."""
        w, bs = self.w, self.w.block_size
        for rid, n in cached_tokens(w):
            blocks = torch.tensor(self.cb.cb_sched_get_blocks(self.sched, rid), dtype=torch.int64,
                                  device=self.device)
            for a in range(0, n, rows_per_batch):
                b = min(n, a + rows_per_batch)
                pos = torch.arange(a, b, dtype=torch.int64, device=self.device)
                slots = (blocks[pos // bs] * bs + pos % bs).to(torch.int32)
                k = values.token_values(w.seed, "k", rid, pos, w.Hkv, w.D, self.dtype, self.device)
                v = values.token_values(w.seed, "v", rid, pos, w.Hkv, w.D, self.dtype, self.device)
                self.runner.append_rows(pos.to(torch.int32), slots, k, v)
            self.written += n

    def step_inputs(self, meta):
        """Raw q, k, v of the step's rows from the generator, on the device."""
        w = self.w
        h = meta.host
        qlens = (h["cu_seqlens_q"][1:] - h["cu_seqlens_q"][:-1]).long()
        reqs = torch.repeat_interleave(h["seq_ids"].long(), qlens).to(self.device)
        pos = h["positions"].long().to(self.device)
        q = values.rows_values(w.seed, "q", reqs, pos, w.Hq, w.D, self.dtype, self.device)
        k = values.rows_values(w.seed, "k", reqs, pos, w.Hkv, w.D, self.dtype, self.device)
        v = values.rows_values(w.seed, "v", reqs, pos, w.Hkv, w.D, self.dtype, self.device)
        return q, k, v

    def step(self, budget=None, inputs=None):
        """Arrivals, build, copy, rope + append, attention.  Returns (meta, out [T, Hq, D], q_rot)."""
        self.arrive(self.step_index)
        self.step_index += 1
        meta = self.runner.build(self.sched, self.w.budget if budget is None else budget)
        dev = self.runner.upload(meta)
        q, k, v = self.step_inputs(meta) if inputs is None else inputs
        q_rot = torch.empty_like(q)
        out = torch.empty_like(q)
        self.runner.append(dev, q, k, v, q_rot)
        self.runner.attend(meta, dev, q_rot, out)
        self.written += meta.num_tokens
        return meta, out, q_rot

    def cache_rows(self, slots: np.ndarray):
        """(k, v) stored at ``slots``: float32 numpy [n, Hkv, D], plus raw bit patterns."""
        bs = self.w.block_size
        sl = torch.as_tensor(slots, dtype=torch.int64, device=self.device)
        kk = self.runner.k_cache[sl // bs, :, sl % bs, :]
        vv = self.runner.v_cache[sl // bs, :, sl % bs, :]
        ity = torch.int16 if self.dtype == torch.bfloat16 else torch.int32
        return (kk.float().cpu().numpy(), vv.float().cpu().numpy(),
                kk.view(ity).cpu().numpy(), vv.view(ity).cpu().numpy())

    def sentinel_count(self) -> int:
        """Cache elements (K and V) still holding the all-ones sentinel."""
        ity = torch.int16 if self.dtype == torch.bfloat16 else torch.int32
        return int((self.runner.k_cache.view(ity) == -1).sum() + (self.runner.v_cache.view(ity) == -1).sum())
