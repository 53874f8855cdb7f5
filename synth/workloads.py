"""The five synthetic mixed-step workloads and their seeded structure draws.

Shared, as input data only, by the oracle harness and the HIP harness.  Nothing here schedules,
rotates or attends: a workload is a list of running decodes (with the context each already has
in the cache), a FCFS list of prompts, a token budget, a block pool and the head geometry.

Structure draws use ``numpy.random.Generator(PCG64(seed))`` in a fixed order: decode contexts,
then prompt lengths, then the physical free-list permutation.  Contexts are integer-uniform on
inclusive ranges; prompt lengths in the log-normal workload are ``exp(N(ln 6000, 0.5))`` rounded
half-to-even and clipped to ``[1, 16384]``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                  # "f32" or "bf16": storage type of q, k, v, caches and output
    Hq: int
    Hkv: int
    D: int
    block_size: int
    budget: int                 # token budget per step
    decode_ctx: tuple           # tokens already cached for each running decode
    prompts: tuple              # (prompt_len, cached_len) in FCFS order
    num_blocks: int
    free_list: tuple | None     # physical block allocation order; None = 0..num_blocks-1
    steps: int | None           # None: run until every prompt has had its last chunk
    seed: int
    max_steps: int = 64
    arrivals: tuple = ()        # (step, prompt_len, cached_len): prompts joining the queue before
                                # that step's build (0-based), after the ones listed in ``prompts``

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def num_decodes(self) -> int:
        return len(self.decode_ctx)

    def request_ids(self):
        """Request indices: decodes 0..nd-1 in order, then prompts in FCFS order."""
        nd = len(self.decode_ctx)
        return list(range(nd)), list(range(nd, nd + len(self.prompts)))

    def max_position(self) -> int:
        """An upper bound on any absolute position the run can touch."""
        s = self.max_steps if self.steps is None else self.steps
        m = max([c + s for c in self.decode_ctx] + [L + s for L, _ in self.prompts] +
                [L + s for _, L, _ in self.arrivals] + [1])
        return m + 1

    def arriving(self, step: int):
        """(prompt_len, cached_len) of the prompts that join the queue before ``step``'s build."""
        return [(L, c) for t, L, c in self.arrivals if t == step]


def _pool_size(decode_ctx, prompts, bs, steps) -> int:
    n = sum(-(-(c + steps) // bs) for c in decode_ctx)
    n += sum(-(-(L + steps) // bs) for L, _ in prompts)
    return n + 8


def _make(name, dtype, Hq, Hkv, D, bs, budget, decode_ctx, prompts, steps, seed, rng,
          identity_free_list=False, max_steps=64):
    decode_ctx = tuple(int(c) for c in decode_ctx)
    prompts = tuple((int(L), int(c)) for L, c in prompts)
    s = max_steps if steps is None else steps
    nb = _pool_size(decode_ctx, prompts, bs, s)
    free = None if identity_free_list else tuple(int(b) for b in rng.permutation(nb))
    return Workload(name, dtype, Hq, Hkv, D, bs, budget, decode_ctx, prompts, nb, free, steps,
                    seed, max_steps)


def config1() -> Workload:
    """Budget-8 worked example: 3 decodes (16/20/24 cached) and one 12-token prompt, fp32."""
    rng = np.random.Generator(np.random.PCG64(1001))
    return _make("cfg1_worked_example_f32", "f32", 4, 4, 64, 16, 8, (16, 20, 24), ((12, 0),),
                 4, 1001, rng, identity_free_list=True)


def config2() -> Workload:
    """7B-like layer: 32/32 heads, D 128, block 16; 64 decodes U{512..4096}; 4096 prompt; B 512."""
    rng = np.random.Generator(np.random.PCG64(1002))
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return _make("cfg2_7b_b512_bf16", "bf16", 32, 32, 128, 16, 512, ctx, ((4096, 0),), 10,
                 1002, rng)


def config3() -> Workload:
    """13B-like layer: 40/40 heads; 32 decodes at 2048; one 4096 prompt; B 544 (C = 512)."""
    rng = np.random.Generator(np.random.PCG64(1003))
    return _make("cfg3_13b_b544_bf16", "bf16", 40, 40, 128, 16, 544, [2048] * 32, ((4096, 0),),
                 9, 1003, rng)


def config4() -> Workload:
    """GQA 34B-like layer: 56/8 heads; 128 decodes U{1024..8192}; 8 log-normal prompts; B 2048."""
    rng = np.random.Generator(np.random.PCG64(1004))
    ctx = rng.integers(1024, 8192, size=128, endpoint=True)
    z = rng.normal(math.log(6000.0), 0.5, size=8)
    lens = np.clip(np.rint(np.exp(z)), 1, 16384).astype(np.int64)
    return _make("cfg4_gqa34b_b2048_bf16", "bf16", 56, 8, 128, 16, 2048, ctx,
                 tuple((int(L), 0) for L in lens), None, 1004, rng, max_steps=64)


def config5() -> Workload:
    """Long context: 64/8 heads, block 32; 256 decodes U{1024..32768}; a 2048-token chunk after
    a 262,144-token cached prefix; B 8192."""
    rng = np.random.Generator(np.random.PCG64(1005))
    ctx = rng.integers(1024, 32768, size=256, endpoint=True)
    return _make("cfg5_longctx_b8192_bf16", "bf16", 64, 8, 128, 32, 8192, ctx,
                 ((262144 + 2048, 262144),), 1, 1005, rng)


BUILDERS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def stream_b512() -> Workload:
    """Serving-like traffic on the budget-512 layer's geometry (32/32 heads, D 128, block 16): 64
    decodes U{512..4096} and 16 prompts arriving over a 48-step cycle (exponential gaps of mean 2.5
    steps, log-normal lengths of median 300, sigma 0.8, cap 1500, nothing cached), so the token
    count and the decode count change from step to step."""
    from synth.streams import mixed_stream
    rng = np.random.Generator(np.random.PCG64(1012))
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    reqs = mixed_stream(1012, 16, mean_gap=2.5, median_prompt=300, sigma=0.8, max_prompt=1500)
    arrivals = tuple((r.arrival - 1, r.prompt_len, 0) for r in reqs)
    steps = 48
    nb = _pool_size(ctx, [(L, 0) for _, L, _ in arrivals], 16, steps)
    free = tuple(int(b) for b in rng.permutation(nb))
    return Workload("stream_b512_bf16", "bf16", 32, 32, 128, 16, 512, tuple(int(c) for c in ctx), (), nb,
                    free, steps, 1012, steps, arrivals)


def get(i: int) -> Workload:
    return BUILDERS[i]()


def small(i: int) -> Workload:
    """Scaled-down variants of the five workloads (same structure and draws, fewer heads and
    tokens) that the oracle checks row by row in seconds while spanning several query tiles,
    several key tiles and ragged tails."""
    rng = np.random.Generator(np.random.PCG64(2000 + i))
    if i == 1:
        return config1()
    if i == 2:   # MHA, 6 decodes, one prompt in 294-token chunks (3 query tiles), 5 steps
        ctx = rng.integers(100, 700, size=6, endpoint=True)
        return _make("small2_mha_bf16", "bf16", 4, 4, 128, 16, 300, ctx, ((1200, 0),), 5, 2002, rng)
    if i == 3:   # 5 heads, decodes at 300, C = 128
        return _make("small3_mha_bf16", "bf16", 5, 5, 128, 16, 132, [300] * 4, ((600, 0),), 6,
                     2003, rng)
    if i == 4:   # GQA group of 7, three prompts, several chunks per step
        ctx = rng.integers(100, 900, size=8, endpoint=True)
        z = rng.normal(math.log(400.0), 0.5, size=3)
        lens = np.clip(np.rint(np.exp(z)), 1, 1200).astype(np.int64)
        return _make("small4_gqa7_bf16", "bf16", 14, 2, 128, 16, 256, ctx,
                     tuple((int(L), 0) for L in lens), None, 2004, rng, max_steps=32)
    if i == 5:   # GQA group of 8, block 32, chunk of 500 after a 3000-token cached prefix
        ctx = rng.integers(100, 3000, size=8, endpoint=True)
        return _make("small5_gqa8_longctx_bf16", "bf16", 16, 2, 128, 32, 1024, ctx,
                     ((3500, 3000),), 1, 2005, rng)
    if i == 6:   # head dim 64 in bf16
        ctx = rng.integers(20, 400, size=5, endpoint=True)
        return _make("small6_d64_bf16", "bf16", 4, 2, 64, 16, 200, ctx, ((500, 0),), 3, 2006, rng)
    if i == 7:   # float32 at head dim 128
        ctx = rng.integers(20, 300, size=4, endpoint=True)
        return _make("small7_d128_f32", "f32", 4, 4, 128, 16, 160, ctx, ((400, 0),), 3, 2007, rng)
    if i == 9:   # arrivals: 4 decodes, prompts joining at steps 0, 1, 3 and 4 (the token and
        # decode counts change from step to step)
        ctx = rng.integers(100, 600, size=4, endpoint=True)
        nb = _pool_size(ctx, [(300, 0), (90, 0), (170, 40), (60, 0)], 16, 8)
        return Workload("small9_arrivals_bf16", "bf16", 8, 2, 128, 16, 128, tuple(int(c) for c in ctx), (),
                        nb, tuple(int(b) for b in rng.permutation(nb)), 8, 2009, 8,
                        ((0, 300, 0), (1, 90, 0), (3, 170, 40), (4, 60, 0)))
    if i == 8:   # decode-heavy: 24 decodes U{1500..3000} x 16 heads, ~27K 32-key decode stages,
        # so the stage split spreads each unit over several waves and the combine merges several
        # partials per row and head
        ctx = rng.integers(1500, 3000, size=24, endpoint=True)
        return _make("small8_decode_tail_bf16", "bf16", 16, 16, 128, 16, 324, ctx, ((600, 0),), 3,
                     2008, rng)
    raise KeyError(i)


SMALL = (1, 2, 3, 4, 5, 6, 7, 8, 9)
