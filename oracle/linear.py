"""Linear layers around the attention step (oracle; test infrastructure only).

What it follows: "Chunked Prefill: Ending the Great Stall" §02 (selective batching: the linear
layers of an iteration run over the tokens of every request in it, decode and prefill alike) and
"Splitting Prefill From Decode Inside a Step" ("Two kernels with different limiting resources":
the weights are read once per step and a step of T tokens performs about 2 N T operations for
N parameters).  The layer is the plain definition

    y[t, n] = sum_k x[t, k] * w[n, k]

evaluated in fp64 from the stored (bf16) values; weights are laid out [out_features,
in_features] (this implementation's choice; the pages fix none).  ``bound`` gives, per element,
a rigorous bound on how far a float32-accumulated result rounded once to bfloat16 can lie from it.
"""
from __future__ import annotations

import numpy as np

BF16_HALF_ULP = 2.0 ** -8       # relative rounding error of round-to-nearest into bfloat16
F32_UNIT = 2.0 ** -24           # unit roundoff of float32


def linear(x, w) -> np.ndarray:
    """x [M, K], w [N, K] (any float type, widened exactly) -> x . w^T in fp64 [M, N]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError("inner dimensions differ")
    return x @ w.T


def bound(x, w) -> np.ndarray:
    """Per-element bound on |bf16(fl32 sum) - exact| for any float32 summation order:
    gamma_K * sum_k |x w| for the accumulation (Higham, "Accuracy and Stability of Numerical
    Algorithms", 2nd ed., §3.1, with gamma_K = K u / (1 - K u)) plus the final rounding's half ulp
    of the accumulated value."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = x.shape[1]
    gamma = K * F32_UNIT / (1.0 - K * F32_UNIT)
    acc = gamma * (np.abs(x) @ np.abs(w).T)           # float32 accumulation error, any order
    # The accumulated value s satisfies |s| <= |exact| + acc; rounding it to bf16 moves it by at
    # most half an ulp of |s|.
    return BF16_HALF_ULP * (np.abs(linear(x, w)) + acc) + acc


def flops(T: int, K: int, N: int) -> int:
    """Multiply-adds of one layer over T tokens, counted as 2 operations each."""
    return 2 * T * K * N
