"""Full-prefill causal attention in fp64, and the expected paged-cache contents (oracle; test only).

What it follows:

* Chunked Prefill 的 Token 预算 (zwjcode), §02: a query at position i depends only on keys and
  values 0..i, so processing a prompt in order, piece by piece, equals processing it at once; §07:
  a query at row i of a chunk that starts at offset c sees keys {0, ..., c + i} (the cached prefix
  plus its own chunk up to itself), not only c..c+i.
* Chunked Prefill: Ending the Great Stall (manishklach), §05: the attention of a chunk is an
  ordinary causal attention over every earlier token plus the chunk; paged blocks are filled
  token-sequentially, so chunk boundaries are invisible to the cache.

So the oracle never chunks: for every requested row of sequence s at absolute position p and
query head h it evaluates, in fp64 with an exact two-pass softmax,

    out[p, h] = sum_{j=0..p} softmax_j( (q^_p,h . k^_j,g) * scale ) * v_j,g,   g = h // (Hq / Hkv)

where q^ and k^ are the rotated vectors rounded into the storage type and v is the stored value.
Reading used (the pages are silent): scale = 1 / sqrt(D), contiguous query-head groups per KV head,
no window, bias or soft cap.
"""
from __future__ import annotations

import numpy as np


def attend(q_hat: np.ndarray, k_hat: np.ndarray, v: np.ndarray, positions, scale: float,
           row_block: int = 128) -> np.ndarray:
    """Causal attention of rows of ONE sequence over that sequence's keys.

    q_hat:     [R, Hq, D]  rotated queries (any float type; promoted to fp64)
    k_hat, v:  [P, Hkv, D] rotated keys and values for positions 0..P-1 of the sequence
    positions: [R] absolute position of each row; each must be < P
    returns    [R, Hq, D] float64
    """
    q_hat = np.asarray(q_hat, dtype=np.float64)
    R, Hq, D = q_hat.shape
    P, Hkv, _ = k_hat.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    pos = np.asarray(positions, dtype=np.int64)
    if R and int(pos.max()) >= P:
        raise ValueError("a row's position lies beyond the supplied keys")
    out = np.empty((R, Hq, D), dtype=np.float64)
    for r0 in range(0, R, row_block):
        pr = pos[r0:r0 + row_block]
        nk = int(pr.max()) + 1
        keys = np.arange(nk)
        hidden = keys[None, :] > pr[:, None]                         # [r, nk] keys after the row
        for g in range(Hkv):
            kg = np.asarray(k_hat[:nk, g, :], dtype=np.float64)       # [nk, D]
            vg = np.asarray(v[:nk, g, :], dtype=np.float64)
            qg = q_hat[r0:r0 + row_block, g * G:(g + 1) * G, :]       # [r, G, D]
            s = np.matmul(qg, kg.T) * scale                           # [r, G, nk]
            s = np.where(hidden[:, None, :], -np.inf, s)
            m = s.max(axis=-1, keepdims=True)                         # pass 1: max
            e = np.exp(s - m)
            den = e.sum(axis=-1, keepdims=True)                       # pass 2: sum
            out[r0:r0 + row_block, g * G:(g + 1) * G, :] = np.matmul(e, vg) / den
    return out


def expected_slots(slot_mapping, values: np.ndarray, block_size: int):
    """Where each token's K (or V) must sit in a [num_blocks, Hkv, block_size, D] cache.

    Returns (block index [n], offset in block [n], values [n, Hkv, D]) for tokens with slot >= 0.
    The cache layout is this implementation's choice; the rule that a token at slot
    ``block * block_size + offset`` lands in that block at that offset is the pages' (zwjcode §06:
    slot_mapping names the physical slot of each new K/V).
    """
    sm = np.asarray(slot_mapping, dtype=np.int64)
    keep = sm >= 0
    return sm[keep] // block_size, sm[keep] % block_size, np.asarray(values)[keep]
