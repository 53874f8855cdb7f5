"""One mixed step on one GPU: build (C++), metadata pull (kernel), rope + append, attention.

``MixedStepRunner`` owns the device side of a serving layer for one head geometry: the paged
K/V caches (``[num_blocks, Hkv, block_size, D]``), the rotary table, a ring of two pinned
metadata buffers, the device copy of the metadata and the attention workspace.  Each call below
forwards to one C entry point of libcb.so; the runner only allocates and orders them on the
current torch stream.

The host stays at most two steps ahead of the device (the pinned-buffer ring), so a host stall
longer than two steps' device time leaves the GPU idle.  Python's cyclic collector is one: a pass
over a process's long-lived objects takes about a millisecond.  A serving loop should
``gc.collect(); gc.freeze()`` once its set-up is done, as ``bench.py`` does.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import binding as cb

SENTINEL_BITS = {torch.bfloat16: -1, torch.float32: -1}   # all-ones: a NaN that no write produces


class HipEvent:
    """A HIP event recorded without the system-scope fence (the runtime's
    hipEventDisableSystemFence), with or without timing.

    A default event's record ends in a system-scope release: a writeback of the device's caches
    before the event completes, which the work behind it waits for.  Neither use here needs it:
    the pull marks (``MixedStepRunner.mark_pulled``) only tell the host that a pull kernel has
    read its pinned buffer -- no device write has to become visible to the host -- and timing
    events only take timestamps.  Measured on the budget-512 step loop: 420.1 us per step with a
    default event after each pull, 418.5-418.7 with this one.  Duck-typed as ``torch.cuda.Event``
    for ``record``, ``synchronize``, ``elapsed_time`` and ``cuda_event`` (the handle the timed
    attention call records).  The calls go to the HIP runtime libcb.so is linked against, through
    its handle."""

    _DISABLE_TIMING, _NO_SYSTEM_FENCE = 0x2, 0x20000000
    _SIGS = (("hipEventCreateWithFlags", [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]),
             ("hipEventRecord", [ctypes.c_void_p, ctypes.c_void_p]),
             ("hipEventSynchronize", [ctypes.c_void_p]),
             ("hipEventElapsedTime", [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]),
             ("hipEventDestroy", [ctypes.c_void_p]))

    def __init__(self, timing: bool = False):
        hip = cb._lib()
        for name, args in self._SIGS:
            fn = getattr(hip, name)
            fn.restype, fn.argtypes = ctypes.c_int, args
        self._hip = hip
        self._ev = ctypes.c_void_p()
        flags = self._NO_SYSTEM_FENCE | (0 if timing else self._DISABLE_TIMING)
        self._call("hipEventCreateWithFlags", ctypes.byref(self._ev), flags)

    def _call(self, name, *args):
        rc = getattr(self._hip, name)(*args)
        if rc != 0:
            raise RuntimeError(f"{name} failed with HIP error {rc}")

    @property
    def cuda_event(self) -> int:
        return self._ev.value

    def record(self, stream: torch.cuda.Stream | None = None):
        if stream is None:
            stream = torch.cuda.current_stream()
        self._call("hipEventRecord", self._ev, ctypes.c_void_p(stream.cuda_stream))

    def synchronize(self):
        self._call("hipEventSynchronize", self._ev)

    def elapsed_time(self, end: "HipEvent") -> float:
        """Milliseconds from this event to ``end`` (both recorded with timing and complete)."""
        ms = ctypes.c_float()
        self._call("hipEventElapsedTime", ctypes.byref(ms), self._ev, end._ev)
        return ms.value

    def __del__(self):
        ev = getattr(self, "_ev", None)
        if ev is not None and ev.value:
            try:
                self._hip.hipEventDestroy(ev)
            except Exception:       # interpreter shutdown
                pass


def round_up(x: int, step: int) -> int:
    return -(-x // step) * step if step > 0 else x


class Buckets:
    """Padded launch shapes, so that steps whose exact shapes differ share one captured graph.

    A step's launches take its token count and its longest query and contexts by value; rounding
    them up gives a handful of keys instead of one per step.  The token count rounds up to a
    multiple of ``tokens`` (at most the buffers' capacity): the padding rows get position and slot
    -1, which the rotary/append kernel skips, and their attention output is left undefined.  The
    longest query rounds up to a multiple of ``tokens`` too (it sizes the chunk tiles' query
    blocks) and the longest contexts to a multiple of ``context`` (they size the grids and the
    workspace); the kernels read each row's own lengths from the metadata, so larger bounds only
    add tiles that exit at once and may choose other key splits.  The sequence and decode counts
    stay exact: padding them would need dummy rows inside the metadata.
    """

    def __init__(self, tokens: int = 64, context: int = 4096):
        self.tokens, self.context = tokens, context


class MixedStepRunner:
    def __init__(self, *, Hq: int, Hkv: int, D: int, block_size: int, num_blocks: int,
                 dtype: torch.dtype, device, max_pos: int, cap_seqs: int, cap_tokens: int,
                 cap_blocks: int, sentinel: bool = True, rope_base: float = 10000.0):
        self.Hq, self.Hkv, self.D, self.bs = Hq, Hkv, D, block_size
        self.dtype = dtype
        self.device = torch.device(device)
        self.scale = 1.0 / math.sqrt(D)
        shape = (num_blocks, Hkv, block_size, D)
        self.k_cache = torch.empty(shape, dtype=dtype, device=self.device)
        self.v_cache = torch.empty(shape, dtype=dtype, device=self.device)
        if sentinel:
            ity = torch.int16 if dtype == torch.bfloat16 else torch.int32
            self.k_cache.view(ity).fill_(SENTINEL_BITS[dtype])
            self.v_cache.view(ity).fill_(SENTINEL_BITS[dtype])
        self.cos_sin = cb.cb_rope_cos_sin(max_pos, D, rope_base).to(self.device)
        # The decode rows' work split is made on the host after each build (cb_decode_plan) and
        # travels with the metadata, so the attention call launches no split kernel.
        self.plan_waves = {h: cb.cb_attn_decode_waves(self.device, h) for h in (False, True)}
        plan_ints = cb.cb_decode_plan_ints(cap_seqs, max(self.plan_waves.values()))
        # Two pinned host buffers and two device buffers.  Step n's metadata is pulled onto the
        # device by a kernel on the compute stream (so device buffer i is rewritten in stream
        # order); host buffer i is rewritten (step n + 2) only after that kernel has finished.
        self.bufs = [cb.StepBuffers(cap_seqs, cap_tokens, cap_blocks, plan_ints=plan_ints) for _ in range(2)]
        self.dev_flat = [torch.empty_like(b.flat, device=self.device) for b in self.bufs]
        self.marks = [None, None]                  # HipEvents, made at the first pull (host-only use needs none)
        self.copied = [None, None]                 # mark of the last pull from host buffer i
        self.ring = 0
        self.workspace = torch.empty(0, dtype=torch.uint8, device=self.device)

    # ---- host builder + metadata copy ----------------------------------------------------------
    def build(self, sched: cb.Sched, budget: int, buckets: Buckets | None = None) -> cb.StepMeta:
        """cb_build_step into the next pinned buffer (after its previous copy has finished).  With
        ``buckets`` the launch shape is padded (``meta.launch_tokens`` rows and rounded-up maxima;
        see ``Buckets``) before the decode split is planned for it."""
        i = self.ring
        self.ring ^= 1
        if self.copied[i] is not None:
            self.copied[i].synchronize()
        meta = cb.cb_build_step(sched, budget, self.bufs[i])
        if meta.max_context_len > self.cos_sin.shape[0]:
            # cb_rope_kv_append skips rows beyond the rotary table (its padding convention), which
            # would leave their K/V unwritten and their queries unrotated: stop instead.  The
            # builder has already committed the step, so this is fatal for the serving loop (it
            # was configured with too small a max_pos).
            raise ValueError(f"step reaches position {meta.max_context_len - 1}, beyond the rotary table's "
                             f"{self.cos_sin.shape[0]} rows (max_pos)")
        meta.buf_index = i
        meta.plan_waves = 0
        meta.launch_tokens = meta.num_tokens
        if buckets is not None:
            self._pad(meta, buckets)
        nd = meta.num_decodes
        if nd > 0:
            S = meta.num_seqs
            meta.plan_waves = cb.cb_decode_plan(meta.host["cu_seqlens_q"][:S + 1], meta.host["context_lens"][:S],
                                                nd, meta.max_q_len, meta.max_context_len, self.Hq, self.Hkv,
                                                self.bufs[i].arrays["decode_plan"], self.device)
        return meta

    def _pad(self, meta: cb.StepMeta, b: Buckets):
        T = meta.num_tokens
        cap = self.bufs[meta.buf_index].cap[1]
        Tp = min(cap, round_up(T, b.tokens))
        arrays = self.bufs[meta.buf_index].arrays
        arrays["positions"][T:Tp] = -1              # padding rows: skipped by the append
        arrays["slot_mapping"][T:Tp] = -1
        meta.launch_tokens = Tp
        meta.exact_max = (meta.max_q_len, meta.max_context_len, meta.max_decode_context_len)
        meta.max_q_len = min(round_up(meta.max_q_len, b.tokens), Tp)
        meta.max_context_len = round_up(meta.max_context_len, b.context)
        meta.max_decode_context_len = round_up(meta.max_decode_context_len, b.context)

    def upload(self, meta: cb.StepMeta) -> dict:
        """cb_copy_host_to_device of the step's metadata on the current stream (a kernel, so the
        kernels that follow need no cross-queue wait).  Returns device int32 views."""
        dev = self.pull(meta)
        self.mark_pulled(meta)
        return dev

    def pull(self, meta: cb.StepMeta) -> dict:
        """The metadata-pull kernel alone (device work only; see upload)."""
        i = meta.buf_index
        buf, dev = self.bufs[i], self.dev_flat[i]
        cb.cb_copy_host_to_device(buf.flat, dev, stream=torch.cuda.current_stream(self.device))
        views = {k: dev[buf.offsets[k]:buf.offsets[k] + n] for k, n in meta.lengths().items()}
        views["decode_plan"] = dev[buf.offsets["decode_plan"]:]
        return views

    def mark_pulled(self, meta: cb.StepMeta):
        """Record that the pinned buffer of ``meta`` may be rewritten once the stream gets here.
        (A mark re-recorded before anyone waited for it only moves later in the stream, which
        keeps the wait in ``build`` correct.)"""
        mark = self.marks[meta.buf_index]
        if mark is None:
            mark = self.marks[meta.buf_index] = HipEvent()
        mark.record(torch.cuda.current_stream(self.device))
        self.copied[meta.buf_index] = mark

    # ---- device work ---------------------------------------------------------------------------
    def append(self, dev: dict, q, k, v, q_out):
        """cb_rope_kv_append: rotate q into q_out, rotate k and append k, v at the step's slots."""
        cb.cb_rope_kv_append(q, k, v, dev["positions"], dev["slot_mapping"], self.cos_sin, q_out,
                             self.k_cache, self.v_cache)

    def append_rows(self, positions, slots, k, v):
        """Append rows outside a step (cache set-up for contexts that already exist)."""
        cb.cb_rope_kv_append(None, k, v, positions, slots, self.cos_sin, None, self.k_cache, self.v_cache)

    def ensure_workspace(self, nbytes: int):
        if self.workspace.numel() < nbytes:
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)

    def workspace_bytes(self, meta: cb.StepMeta) -> int:
        return cb.cb_attn_workspace_bytes(meta.num_seqs, meta.num_decodes, meta.launch_tokens,
                                          meta.max_q_len, meta.max_decode_context_len,
                                          meta.max_context_len, self.Hq, self.Hkv, self.D)

    def attend(self, meta: cb.StepMeta, dev: dict, q_rot, out, events=None):
        """cb_mixed_paged_attention over the step's varlen batch."""
        self.ensure_workspace(self.workspace_bytes(meta))
        cb.cb_mixed_paged_attention(
            q_rot, self.k_cache, self.v_cache, dev["cu_seqlens_q"], dev["context_lens"],
            dev["cu_blocks"], dev["block_table"], out, self.workspace,
            num_seqs=meta.num_seqs, num_decodes=meta.num_decodes, max_q_len=meta.max_q_len,
            max_decode_ctx=meta.max_decode_context_len, max_ctx=meta.max_context_len,
            scale=self.scale, events=events,
            decode_plan=dev["decode_plan"] if getattr(meta, "plan_waves", 0) else None,
            plan_waves=getattr(meta, "plan_waves", 0))


class StepGraphs:
    """Whole steps (metadata pull, rope + append, attention) replayed from HIP graphs.

    A captured step bakes in every pointer and every scalar its launches take (token count,
    sequence counts, the longest query and context, the split plan), so a graph serves exactly the
    steps whose launch parameters equal those it was captured with: ``key(meta)`` below, plus the
    pinned buffer the step was built into (the pull reads it by address).  The caller keeps the
    step's device tensors (inputs, q_rot, out) at fixed addresses per key and sizes the workspace
    before the first capture (a reallocation drops every graph).  The first step with a new key
    runs eagerly once (the capture's warm-up) and is then captured; later ones replay.  No timing
    events are recorded inside a graph, and nothing in the captured work clears memory with a
    memset.
    """

    def __init__(self, runner: MixedStepRunner):
        self.runner = runner
        self.graphs = {}
        self.workspace_ptr = None
        self.side = torch.cuda.Stream(device=runner.device)

    @staticmethod
    def key(meta: cb.StepMeta) -> tuple:
        return (meta.buf_index, meta.num_seqs, meta.num_decodes, meta.launch_tokens, meta.max_q_len,
                meta.max_context_len, meta.max_decode_context_len)

    def step(self, meta: cb.StepMeta, launch) -> str:
        """Run ``launch(dev)`` -- the step's device work after the pull, given the device views --
        for ``meta``: replayed when a graph for its key exists, else eagerly and then captured.
        Returns "replay" or "captured"."""
        r = self.runner
        if self.workspace_ptr != r.workspace.data_ptr():
            self.graphs.clear()
            self.workspace_ptr = r.workspace.data_ptr()
        k = self.key(meta)
        g = self.graphs.get(k)
        cur = torch.cuda.current_stream(r.device)
        if g is not None:
            g.replay()
            r.mark_pulled(meta)
            return "replay"
        launch(r.pull(meta))                       # eager run (also the capture's warm-up)
        r.mark_pulled(meta)
        g = torch.cuda.CUDAGraph()
        self.side.wait_stream(cur)
        with torch.cuda.graph(g, stream=self.side):
            launch(r.pull(meta))
        cur.wait_stream(self.side)
        self.graphs[k] = g
        return "captured"
