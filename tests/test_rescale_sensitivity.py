"""The jumping-score inputs of tests/test_gpu_rescale.py can see a wrong rescale.

CPU only.  For chunk rows of each pattern (positions 2,000-2,599) a stage-wise online softmax over
32-key stages with a running reference allowed to lag by up to 8 (base-2 units) is run in float64
(weights rounded to float32, as the kernel holds them) with a mistake planted in its rescale — the
output accumulator not rescaled, the running sum not rescaled, or the reference never moved after
the first stage (weights overflow once a row's scores climb 128 above it: the ramps, not the saw)
— and must fail the bfloat16 bar against the oracle's attention on at least one of the rows (the
GPU test checks them all), while the same online softmax without the mistake passes on every row.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import rope as orope
from synth import values
from tests.harness import compare
from tests.test_gpu_rescale import raw_keys, raw_queries, workload

SLACK = 8.0


def online(q, k, v, pos, scale, mistake=None):
    """[Hq, D] output of one row by 32-key stages; q [Hq, D], k/v [P, Hkv, D] float64."""
    Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    c = scale / np.log(2.0)                       # base-2 units
    out = np.zeros((Hq, D))
    for h in range(Hq):
        g = h // G
        m_ref, l, o = -np.inf, 0.0, np.zeros(D)
        for k0 in range(0, pos + 1, 32):
            kk = k[k0:pos + 1][:32, g, :]
            s = kk @ q[h]                          # raw scores of the stage
            cand = s.max() * c
            limit = m_ref + SLACK
            if mistake == "stale_reference" and m_ref != -np.inf:
                limit = np.inf
            if cand > limit:
                m_new = max(m_ref, cand)
                alpha = 0.0 if m_ref == -np.inf else 2.0 ** (m_ref - m_new)
                if mistake != "l_not_rescaled":
                    l *= alpha
                if mistake != "o_not_rescaled":
                    o *= alpha
                m_ref = m_new
            with np.errstate(over="ignore"):
                p = np.float32(2.0) ** (s * c - (m_ref if m_ref != -np.inf else 0.0)).astype(np.float32)
            p = p.astype(np.float64)
            l += p.sum()
            o += p @ v[k0:pos + 1][:32, g, :]
        out[h] = o / l
    return out


@pytest.mark.parametrize("pattern", ["steep", "gentle", "saw"])
def test_planted_rescale_mistakes_fail_the_bar(pattern):
    w = workload()
    P = 2600
    rows = np.arange(2000, P, 75).tolist() + [P - 1]
    table = orope.cos_sin_table(w.max_position(), w.D)
    kpos = np.arange(P)
    kh = orope.rotate_stored(raw_keys(pattern, kpos, w.Hkv, w.D), kpos, table, w.dtype).astype(np.float64)
    v = values.token_values(w.seed, "v", len(w.decode_ctx), torch.as_tensor(kpos), w.Hkv, w.D,
                            torch.bfloat16, "cpu").float().numpy().astype(np.float64)
    qh = orope.rotate_stored(raw_queries(len(rows), w.Hq, w.D), np.array(rows), table, w.dtype).astype(np.float64)
    scale = w.D ** -0.5
    want = oattn.attend(qh, kh, v, rows, scale)
    for i, pos in enumerate(rows):
        assert compare(online(qh[i], kh, v, pos, scale).astype(np.float32), want[i], "bf16")[0], pos
    mistakes = ["o_not_rescaled", "l_not_rescaled"] + (["stale_reference"] if pattern != "saw" else [])
    for mistake in mistakes:
        caught = 0
        for i, pos in enumerate(rows):
            with np.errstate(invalid="ignore", over="ignore"):
                got = online(qh[i], kh, v, pos, scale, mistake)
            got = np.nan_to_num(got, nan=1e30, posinf=1e30, neginf=-1e30).astype(np.float32)
            caught += not compare(got, want[i], "bf16")[0]
        assert caught > 0, f"{pattern}: {mistake} passes the bar on every row"
