"""Seeded request streams for the step simulator (input data only: nothing here schedules).

A stream is a list of requests, each with the step it arrives at, its prompt length, the part of
the prompt already cached and the number of output tokens it generates.  Draws use
``numpy.random.Generator(PCG64(seed))`` in a fixed order: inter-arrival gaps, prompt lengths,
cache hits, output lengths.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Request:
    arrival: int         # step (1-based) at whose start the request joins the queue
    prompt_len: int
    cached_len: int      # tokens of the prompt already cached (0 <= cached_len < prompt_len)
    output_len: int      # tokens generated, the first one by the step that runs the prompt's end


def mixed_stream(seed: int, n: int, mean_gap: float = 2.0, median_prompt: int = 1500,
                 sigma: float = 1.0, max_prompt: int = 32768, hit_rate: float = 0.0,
                 mean_output: int = 64) -> list[Request]:
    """Poisson arrivals (exponential gaps of ``mean_gap`` steps, rounded down), log-normal prompt
    lengths exp(N(ln median_prompt, sigma)) rounded half-even and clipped to [1, max_prompt], a
    cached share drawn uniformly in [0, hit_rate) of each prompt (rounded down, at most
    prompt_len - 1), geometric output lengths with mean ``mean_output``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    gaps = np.floor(rng.exponential(mean_gap, size=n)).astype(np.int64)
    lens = np.clip(np.rint(np.exp(rng.normal(math.log(median_prompt), sigma, size=n))), 1, max_prompt).astype(np.int64)
    hits = rng.uniform(0.0, hit_rate, size=n) if hit_rate > 0 else np.zeros(n)
    outs = rng.geometric(1.0 / mean_output, size=n).astype(np.int64)
    out, t = [], 1
    for i in range(n):
        t += int(gaps[i])
        L = int(lens[i])
        c = min(int(hit_rate and math.floor(hits[i] * L)), L - 1)
        out.append(Request(t, L, c, int(outs[i])))
    return out
