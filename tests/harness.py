"""Drives the HIP path (libcb.so through the binding) and the oracle side by side on one workload.

Both sides take their inputs from ``synth`` only: request structure from ``synth.workloads`` and
activations from ``synth.values`` (raw q/k/v per (request, position)).  Nothing computed by the HIP
path is ever fed to the oracle.  Raw values for the oracle may be generated on the GPU by
``synth`` (torch integer ops) for speed and copied to the host: they are generator output, not
results of the HIP path.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import attention as oattn
from oracle import rope as orope
from oracle.builder import RefBuilder
from synth import values, workloads
from tests.gpu_harness import TORCH_DTYPE, DeviceRun, cached_tokens, step_caps  # noqa: F401

TOL = {"f32": (1e-4, 0.0), "bf16": (2e-2, 1e-2)}        # (atol, rtol)


# ---------------------------------------------------------------------------------------------
# Oracle side
# ---------------------------------------------------------------------------------------------
class OracleRun:
    def __init__(self, w: workloads.Workload, value_device="cpu", sched_cfg: dict | None = None):
        self.w = w
        self.b = RefBuilder(w.block_size, w.num_blocks, w.free_list, **(sched_cfg or {}))
        for c in w.decode_ctx:
            self.b.add_running(c)
        for L, cached in w.prompts:
            self.b.add_prompt(L, cached)
        self.table = orope.cos_sin_table(w.max_position(), w.D)
        self.scale = 1.0 / math.sqrt(w.D)
        self.value_device = value_device
        self.build_index = 0

    def raw(self, tensor: str, rid: int, pos) -> np.ndarray:
        n_heads = self.w.Hq if tensor == "q" else self.w.Hkv
        x = values.token_values(self.w.seed, tensor, rid, pos, n_heads, self.w.D,
                                dtype=TORCH_DTYPE[self.w.dtype], device=self.value_device)
        return x.float().cpu().numpy()

    def build(self, budget=None) -> dict:
        for L, cached in self.w.arriving(self.build_index):
            self.b.add_prompt(L, cached)
        self.build_index += 1
        return self.b.build(self.w.budget if budget is None else budget)

    def expected_kv(self, rid: int, pos: np.ndarray):
        """(k^, v) in the storage type (as float32) for positions ``pos`` of request ``rid``."""
        k = orope.rotate_stored(self.raw("k", rid, pos), pos, self.table, self.w.dtype)
        v = self.raw("v", rid, pos)
        return k, v

    def expected_kv_rows(self, reqs: np.ndarray, pos: np.ndarray):
        """(k^, v) in the storage type (as float32), [n, Hkv, D], for rows given by (request,
        position) pairs, all at once."""
        w = self.w
        dt = TORCH_DTYPE[w.dtype]
        rq = torch.as_tensor(np.asarray(reqs, dtype=np.int64), device=self.value_device)
        ps = torch.as_tensor(np.asarray(pos, dtype=np.int64), device=self.value_device)
        k = values.rows_values(w.seed, "k", rq, ps, w.Hkv, w.D, dt, self.value_device).float().cpu().numpy()
        v = values.rows_values(w.seed, "v", rq, ps, w.Hkv, w.D, dt, self.value_device).float().cpu().numpy()
        return orope.rotate_stored(k, np.asarray(pos), self.table, w.dtype), v

    def expected_rows(self, plan: dict, rows=None) -> dict:
        """fp64 attention for rows of a step (all rows if ``rows`` is None): {row: [Hq, D]}."""
        cu = plan["cu_seqlens_q"]
        want = set(range(plan["num_tokens"])) if rows is None else set(int(r) for r in rows)
        out = {}
        for s in range(plan["num_seqs"]):
            srows = [r for r in range(cu[s], cu[s + 1]) if r in want]
            if not srows:
                continue
            rid = plan["seq_ids"][s]
            pos = np.array([plan["positions"][r] for r in srows])
            last = int(pos.max()) + 1
            kpos = np.arange(last)
            kh, v = self.expected_kv(rid, kpos)
            qh = orope.rotate_stored(self.raw("q", rid, pos), pos, self.table, self.w.dtype)
            res = oattn.attend(qh, kh, v, pos, self.scale)
            for i, r in enumerate(srows):
                out[r] = res[i]
        return out


def bits_of(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage bit patterns of float32-held values of the storage type."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16).view(np.int16) if dtype == "bf16" else u.view(np.int32)


def plan_of_meta(meta) -> dict:
    """The C builder's step as a dict in the oracle's field names."""
    d = {k: v.tolist() for k, v in meta.host.items()}
    for k in ("num_seqs", "num_decodes", "num_tokens", "num_prefill_tokens", "unused_tokens",
              "max_q_len", "max_context_len", "num_blocks_emitted"):
        d[k] = getattr(meta, k)
    return d


def compare(got: np.ndarray, want: np.ndarray, dtype: str):
    """(pass, max_abs, max_rel) under |got - want| <= atol + rtol |want|."""
    atol, rtol = TOL[dtype]
    err = np.abs(got.astype(np.float64) - want)
    ok = bool(np.all(err <= atol + rtol * np.abs(want))) and bool(np.all(np.isfinite(got)))
    rel = err / np.maximum(np.abs(want), 1e-6)
    return ok, float(err.max(initial=0.0)), float(rel.max(initial=0.0))
