"""Pins for the linear-layer oracle (oracle/linear.py) against closed forms and brute force.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import linear as olin
from oracle.rope import bf16_round
from synth.values import matrix_values


def test_identity_weights_return_the_input():
    x = matrix_values(5, "hidden", 7, 64).numpy()
    assert np.array_equal(olin.linear(x, np.eye(64)), x.astype(np.float64))


def test_rank_one_closed_form():
    # x[t, k] = a_t and w[n, k] = b_n for every k: y[t, n] = K a_t b_n
    a = np.array([0.5, -1.25, 3.0])
    b = np.array([2.0, -0.75])
    K = 64
    y = olin.linear(np.repeat(a[:, None], K, 1), np.repeat(b[:, None], K, 1))
    assert np.array_equal(y, K * a[:, None] * b[None, :])


def test_brute_force_small():
    x = matrix_values(1, "hidden", 3, 5).numpy()
    w = matrix_values(1, "w_o", 4, 5).numpy()
    y = olin.linear(x, w)
    for t in range(3):
        for n in range(4):
            assert y[t, n] == pytest.approx(sum(float(x[t, k]) * float(w[n, k]) for k in range(5)), rel=1e-15, abs=1e-15)


def test_bound_holds_for_a_float32_sum_rounded_to_bf16():
    # A float32 sum in any order, rounded once to bf16, stays within the bound; the bound is not
    # vacuous (a planted error of a few bound-widths breaks it).
    K = 512
    x = bf16_round(matrix_values(2, "hidden", 9, K).numpy())
    w = bf16_round(matrix_values(2, "w_qkv", 11, K, scale=K ** -0.5).numpy())
    exact = olin.linear(x, w)
    lim = olin.bound(x, w)
    rng = np.random.default_rng(0)
    for _ in range(3):
        perm = rng.permutation(K)
        acc = np.zeros((9, 11), dtype=np.float32)
        for k in perm:
            acc = (acc + np.float32(1) * x[:, None, k].astype(np.float32) * w[None, :, k].astype(np.float32)).astype(np.float32)
        got = bf16_round(acc).astype(np.float64)
        assert np.all(np.abs(got - exact) <= lim)
    assert not np.all(np.abs((exact + 4 * lim) - exact) <= lim)


def test_bound_sees_one_bf16_ulp():
    # The final rounding's term scales with the accumulated value, not with sum |x w|: with random
    # signs |exact| ~ sqrt(K) while sum |x w| ~ K.  At a depth where the accumulation term is small
    # (K = 256) an output moved by 1.5 bf16 ulps of the exact value leaves the bound wherever the
    # value is not tiny (a half ulp of |s| is bounded by 2^-8 |s|, up to one ulp at the top of a
    # binade); a rounding term built on sum |x w| would have hidden it.
    K = 256
    x = bf16_round(matrix_values(6, "hidden", 16, K).numpy())
    w = bf16_round(matrix_values(6, "w_qkv", 32, K, scale=K ** -0.5).numpy())
    exact = olin.linear(x, w)
    lim = olin.bound(x, w)
    big = np.abs(exact) > 0.5
    assert big.sum() > 100
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact[big]))) - 7)       # bf16 ulp of each value
    assert np.all(1.5 * ulp > lim[big])
    sabs = olin.linear(np.abs(x), np.abs(w))
    assert np.mean(2.0 ** -8 * sabs[big] > 1.5 * ulp) > 0.9         # the wider term admits most


def test_flops_and_weight_intensity():
    # "Splitting Prefill From Decode Inside a Step": 2 N T operations for N parameters and T tokens;
    # with 2-byte weights read once that is T FLOP per weight byte (512 for a 512-token chunk, the
    # order the manishklach page quotes for its 7B example).
    K, N = 4096, 12288
    assert olin.flops(512, K, N) / (K * N * 2) == 512
    assert olin.flops(1, K, N) == 2 * K * N


def test_matrix_values_are_seeded_and_scaled():
    a = matrix_values(3, "w_o", 16, 32, scale=0.25)
    assert torch.equal(a, matrix_values(3, "w_o", 16, 32, scale=0.25))
    assert not torch.equal(a, matrix_values(3, "w_qkv", 16, 32, scale=0.25))
    assert torch.equal(a, matrix_values(3, "w_o", 16, 32) * 0.25)        # power-of-two scale: exact
    big = matrix_values(4, "hidden", 256, 256)
    assert abs(float(big.mean())) < 0.02 and abs(float(big.std()) - 1) < 0.02
    assert torch.equal(matrix_values(4, "hidden", 8, 256, max_elems=300), big[:8])
