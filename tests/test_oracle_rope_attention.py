"""Pins for the oracle's rotary embedding, bf16 rounding and fp64 attention.  CPU only.

Independent checks: an operation-by-operation float32 emulation (Python doubles rounded to fp32
with ``struct``; double rounding is innocuous for +, -, * since 53 >= 2*24 + 2), torch's bf16
conversion, closed forms and special cases, a pure-Python brute-force softmax, and a chunked
computation written here against the oracle's unchunked one.
"""
import math
import struct

import numpy as np
import pytest
import torch

from oracle import attention, rope
from synth import values
from tests.conftest import golden


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


# ---- rotary table and arithmetic ----------------------------------------------------------

def test_table_first_frequency_is_one_and_position_zero_is_identity():
    t = rope.cos_sin_table(300, 64)
    for p in (0, 1, 2, 17, 299):
        assert t[p, 0] == np.float32(math.cos(p)) and t[p, 32] == np.float32(math.sin(p))
    assert np.all(t[0, :32] == 1) and np.all(t[0, 32:] == 0)
    x = values.range_values(1, "k", 0, 0, 1, 3, 64).numpy()
    assert np.array_equal(rope.rotate(x, np.array([0]), t), x)          # RoPE(., 0) is the identity


def test_table_matches_libm_elementwise():
    D = 128
    t = rope.cos_sin_table(5000, D)
    rng = np.random.default_rng(0)
    for _ in range(2000):
        p, i = int(rng.integers(5000)), int(rng.integers(D // 2))
        th = 10000.0 ** ((-2.0 * i) / D)
        assert t[p, i] == np.float32(math.cos(p * th))
        assert t[p, D // 2 + i] == np.float32(math.sin(p * th))


def test_rotation_matches_operation_by_operation_fp32_emulation():
    D = 16
    t = rope.cos_sin_table(64, D)
    x = values.range_values(5, "q", 2, 0, 40, 2, D).numpy()
    pos = np.arange(40) + 3
    got = rope.rotate(x, pos, t)
    h = D // 2
    for n in range(40):
        for hd in range(2):
            for i in range(h):
                c, s = float(t[pos[n], i]), float(t[pos[n], h + i])
                a, b = float(x[n, hd, i]), float(x[n, hd, h + i])
                o1 = f32(f32(a * c) - f32(b * s))
                o2 = f32(f32(b * c) + f32(a * s))
                assert got[n, hd, i] == np.float32(o1) and got[n, hd, h + i] == np.float32(o2)


def test_rotation_is_a_rotation_by_position_times_frequency():
    # Compare the fp32 rotation with the exact rotation of each pair (i, i + D/2) by p*theta_i.
    D = 128
    t = rope.cos_sin_table(4096, D)
    x = values.range_values(9, "k", 1, 0, 64, 4, D).numpy()
    pos = np.arange(0, 4096, 64)
    got = rope.rotate(x, pos, t).astype(np.float64)
    th = rope.frequencies(D)
    ang = pos[:, None].astype(np.float64) * th[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :64].astype(np.float64), x[..., 64:].astype(np.float64)
    want = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    assert np.max(np.abs(got - want)) < 5e-6
    # relative-position property of the exact rotation: <R(m) q, R(n) k> depends on m - n only
    q, k = x[0, 0].astype(np.float64), x[1, 0].astype(np.float64)

    def rot(v, p):
        a = p * th
        return np.concatenate([v[:64] * np.cos(a) - v[64:] * np.sin(a), v[64:] * np.cos(a) + v[:64] * np.sin(a)])

    assert abs(rot(q, 100) @ rot(k, 40) - rot(q, 1060) @ rot(k, 1000)) < 1e-9
    assert abs(rot(q, 100) @ rot(k, 40) - rot(q, 100) @ rot(k, 41)) > 1e-6


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 5,
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0078125, 3.4e38, -3.4e38, 1e-40,
                  np.inf, -np.inf], dtype=np.float32),
        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32),   # exact ties
    ])
    x = x[np.isfinite(x) | np.isinf(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = rope.bf16_round(x)
    finite = ~np.isnan(want)
    assert np.array_equal(got[finite], want[finite])
    assert np.all(np.isnan(got[~finite]))


# ---- attention ----------------------------------------------------------------------------

def brute_force(q, k, v, pos, scale):
    """Pure-Python softmax attention with explicit exp and sums (tiny inputs only)."""
    R, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros((R, Hq, D))
    for r in range(R):
        for h in range(Hq):
            g = h // G
            sc = [sum(float(q[r, h, d]) * float(k[j, g, d]) for d in range(D)) * scale
                  for j in range(pos[r] + 1)]
            m = max(sc)
            w = [math.exp(s - m) for s in sc]
            tot = sum(w)
            for d in range(D):
                out[r, h, d] = sum(w[j] * float(v[j, g, d]) for j in range(pos[r] + 1)) / tot
    return out


@pytest.mark.parametrize("Hq,Hkv,D,P", [(1, 1, 4, 5), (2, 1, 8, 8), (2, 2, 3, 7)])
def test_attention_matches_brute_force(Hq, Hkv, D, P):
    q = values.range_values(11, "q", 0, 0, P, Hq, D).numpy().astype(np.float64)
    k = values.range_values(11, "k", 0, 0, P, Hkv, D).numpy().astype(np.float64)
    v = values.range_values(11, "v", 0, 0, P, Hkv, D).numpy().astype(np.float64)
    pos = np.arange(P)
    got = attention.attend(q, k, v, pos, 1 / math.sqrt(D))
    want = brute_force(q, k, v, pos, 1 / math.sqrt(D))
    assert np.max(np.abs(got - want)) < 1e-12


def test_special_cases():
    D = 8
    k = values.range_values(2, "k", 0, 0, 6, 2, D).numpy()
    v = values.range_values(2, "v", 0, 0, 6, 2, D).numpy()
    q = values.range_values(2, "q", 0, 0, 6, 2, D).numpy()
    out = attention.attend(q, k, v, np.arange(6), 0.3)
    assert np.array_equal(out[0], v[0].astype(np.float64))              # position 0 sees only v0
    same_k = np.repeat(k[:1], 6, axis=0)
    out = attention.attend(q, same_k, v, np.array([5]), 0.3)[:1]        # equal keys: mean of V
    np.testing.assert_allclose(out[0], v.astype(np.float64).mean(axis=0), atol=1e-15)


def _rotated_prompt(seed, L, Hq, Hkv, D, dtype="f32"):
    t = rope.cos_sin_table(L + 1, D)
    pos = np.arange(L)
    q = rope.rotate_stored(values.range_values(seed, "q", 0, 0, L, Hq, D).numpy(), pos, t, dtype)
    k = rope.rotate_stored(values.range_values(seed, "k", 0, 0, L, Hkv, D).numpy(), pos, t, dtype)
    v = values.range_values(seed, "v", 0, 0, L, Hkv, D).numpy()
    return q, k, v, t


def _chunked_online(q, k, v, split, scale):
    """Chunks in order, each attending the cache written so far plus itself, key by key with an
    online (running max / running sum) softmax -- a different evaluation order from the oracle."""
    L, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((L, Hq, D))
    c = 0
    for d in split:
        for i in range(d):
            p = c + i
            for h in range(Hq):
                g = h // G
                m, s, acc = -np.inf, 0.0, np.zeros(D)
                for j in range(p + 1):                     # sees {0, ..., c + i}
                    x = float(np.dot(q[p, h].astype(np.float64), k[j, g].astype(np.float64))) * scale
                    mn = max(m, x)
                    s = s * math.exp(m - mn) + math.exp(x - mn)
                    acc = acc * math.exp(m - mn) + math.exp(x - mn) * v[j, g].astype(np.float64)
                    m = mn
                out[p, h] = acc / s
        c += d
    return out


def test_chunked_2_3_1_equals_full_prefill():
    g = golden("split_2_3_1.json")
    L = g["prompt_len"]
    q, k, v, _ = _rotated_prompt(21, L, 2, 1, 16)
    full = attention.attend(q, k, v, np.arange(L), 0.25)
    chunked = _chunked_online(q, k, v, g["chunks"], 0.25)
    np.testing.assert_allclose(chunked, full, rtol=g["rtol"], atol=g["atol"])


def test_mutations_are_detected():
    # zwjcode §07: restarting positions at 0 in each chunk, or hiding the cached prefix from a
    # chunk's queries, must change the result.
    g = golden("split_2_3_1.json")
    L, D = g["prompt_len"], 16
    q, k, v, t = _rotated_prompt(21, L, 2, 1, D)
    full = attention.attend(q, k, v, np.arange(L), 0.25)
    # (a) positions reset per chunk
    local = np.concatenate([np.arange(d) for d in g["chunks"]])
    qr = rope.rotate(values.range_values(21, "q", 0, 0, L, 2, D).numpy(), local, t)
    kr = rope.rotate(values.range_values(21, "k", 0, 0, L, 1, D).numpy(), local, t)
    bad = attention.attend(qr, kr, v, np.arange(L), 0.25)
    assert np.max(np.abs(bad - full)) > 1e-3
    # (b) chunk-local visibility {c..c+i}
    bad = np.zeros_like(full)
    c = 0
    for d in g["chunks"]:
        bad[c:c + d] = attention.attend(q[c:c + d], k[c:c + d], v[c:c + d], np.arange(d), 0.25)
        c += d
    assert np.max(np.abs(bad - full)) > 1e-3


def test_visibility_of_the_last_chunk_rows():
    # zwjcode §16 exercise: prompt 10 in [4, 3, 3]; last chunk row i sees keys [0, 7 + i] exactly.
    q, k, v, _ = _rotated_prompt(4, 10, 1, 1, 8)
    for i in range(3):
        row = 7 + i
        base = {row: attention.attend(q[row:row + 1], k, v, [row], 0.35)[0]}
        k2, v2 = k.copy(), v.copy()
        k2[row + 1:] += 3.0
        v2[row + 1:] -= 2.0
        after = attention.attend(q[row:row + 1], k2, v2, [row], 0.35)
        assert np.array_equal(after[0], base[row])                     # later keys invisible
        v3 = v.copy()
        v3[row] += 1.0
        assert not np.array_equal(attention.attend(q[row:row + 1], k, v3, [row], 0.35)[0], base[row])
        v4 = v.copy()
        v4[0] += 1.0                                                   # prefix key 0 is visible
        assert not np.array_equal(attention.attend(q[row:row + 1], k, v4, [row], 0.35)[0], base[row])


def test_row_blocking_does_not_change_the_result():
    q, k, v, _ = _rotated_prompt(8, 300, 4, 2, 16, dtype="bf16")
    a = attention.attend(q, k, v, np.arange(300), 0.25, row_block=128)
    b = attention.attend(q, k, v, np.arange(300), 0.25, row_block=7)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_kv_bytes_per_token_arithmetic():
    g = golden("kv_bytes_13b.json")
    per_token = g["layers"] * g["model_dim"] * 2 * g["bytes_per_elem"]
    assert abs(per_token / 1e6 - g["mb_per_token_approx"]) < 0.05
    per_layer = per_token // g["layers"]
    assert per_layer == 40 * 128 * 2 * 2                  # Hkv * D * (K, V) * bf16 of a 13B layer
    total = g["requests"] * g["tokens_per_request"] * per_token
    assert abs(total / 2**30 - g["gb_total_approx"]) / g["gb_total_approx"] < 0.05


def test_expected_slots_layout():
    blk, off, val = attention.expected_slots([5, -1, 33, 16], np.arange(4)[:, None, None] * np.ones((4, 1, 2)), 16)
    assert list(blk) == [0, 2, 1] and list(off) == [5, 1, 0] and list(val[:, 0, 0]) == [0, 2, 3]
