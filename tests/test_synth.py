"""Pins for the seeded input generator (synth/): SplitMix64 as published, the quantile table, and
independence of chunking.  CPU only."""
import math
import statistics

import numpy as np
import pytest
import torch

from synth import values, workloads

MASK = (1 << 64) - 1


class SequentialSplitMix64:
    """The published sequential SplitMix64 (state += gamma; finalise), in Python big ints."""

    def __init__(self, seed):
        self.x = seed & MASK

    def next(self):
        self.x = (self.x + 0x9E3779B97F4A7C15) & MASK
        z = self.x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
        return z ^ (z >> 31)


def test_splitmix64_known_first_output():
    # Seed 0: the first output of the reference generator is 0xE220A8397B1DCDAF.
    assert SequentialSplitMix64(0).next() == 0xE220A8397B1DCDAF
    got = values.splitmix64_at(0, torch.tensor([0], dtype=torch.int64)).item() & MASK
    assert got == 0xE220A8397B1DCDAF


@pytest.mark.parametrize("seed", [0, 1, 1002, 2**63 + 12345])
def test_counter_form_equals_sequential_generator(seed):
    g = SequentialSplitMix64(seed)
    seq = [g.next() for _ in range(300)]
    ctr = torch.arange(300, dtype=torch.int64)
    got = [(v & MASK) for v in values.splitmix64_at(seed, ctr).tolist()]
    assert got == seq


def test_counter_form_far_counters_match_big_int_math():
    seed = 1005
    ctrs = [0, 1, (1 << 53) - 1, (2 << 52) + 77, 123456789012345]
    for c in ctrs:
        z = (seed + (c + 1) * 0x9E3779B97F4A7C15) & MASK
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK
        z ^= z >> 31
        got = values.splitmix64_at(seed, torch.tensor([c], dtype=torch.int64)).item() & MASK
        assert got == z


def test_quantile_table_properties():
    t = values.quantile_table(torch.float32).double().numpy()
    assert t.shape == (65536,)
    assert np.all(np.diff(t) > 0)
    np.testing.assert_array_equal(t, -t[::-1])            # symmetric quantiles
    nd = statistics.NormalDist()
    for j in (0, 1, 1000, 32767, 32768, 65535):
        assert t[j] == np.float32(nd.inv_cdf((j + 0.5) / 65536))
    assert abs(t.mean()) < 1e-9
    assert 0.999 < t.var() < 1.0                          # discretised N(0,1): slightly below 1


def test_values_are_chunk_independent_and_deterministic():
    whole = values.range_values(7, "k", 3, 0, 50, 2, 16)
    parts = torch.cat([values.range_values(7, "k", 3, a, b, 2, 16)
                       for a, b in [(0, 4), (4, 7), (7, 50)]])
    assert torch.equal(whole, parts)
    assert torch.equal(whole, values.range_values(7, "k", 3, 0, 50, 2, 16))
    other = values.range_values(7, "v", 3, 0, 50, 2, 16)
    assert not torch.equal(whole, other)


def test_value_moments():
    x = values.range_values(1002, "q", 0, 0, 4096, 8, 128).double()
    assert abs(x.mean().item()) < 0.01
    assert abs(x.std().item() - 1.0) < 0.01


def test_bf16_values_are_rounded_fp32_values():
    a = values.range_values(3, "v", 1, 0, 64, 4, 128, dtype=torch.float32)
    b = values.range_values(3, "v", 1, 0, 64, 4, 128, dtype=torch.bfloat16)
    assert torch.equal(a.to(torch.bfloat16), b)


def test_workloads_shapes():
    w1 = workloads.get(1)
    assert w1.decode_ctx == (16, 20, 24) and w1.prompts == ((12, 0),) and w1.budget == 8
    assert w1.free_list is None
    w2 = workloads.get(2)
    assert len(w2.decode_ctx) == 64 and all(512 <= c <= 4096 for c in w2.decode_ctx)
    assert sorted(w2.free_list) == list(range(w2.num_blocks))
    w4 = workloads.get(4)
    assert len(w4.prompts) == 8 and all(1 <= L <= 16384 for L, _ in w4.prompts)
    assert w4.group == 7
    w5 = workloads.get(5)
    assert w5.prompts == ((264192, 262144),) and w5.block_size == 32 and w5.group == 8
    assert workloads.get(2) == w2                           # seeded: identical on every call


def test_rows_values_equal_per_request_values():
    reqs = [0, 0, 3, 7, 3]
    pos = [5, 6, 0, 100, 9]
    got = values.rows_values(17, "k", reqs, pos, 3, 16)
    for i, (r, p) in enumerate(zip(reqs, pos)):
        assert torch.equal(got[i], values.token_values(17, "k", r, [p], 3, 16)[0])
