"""Seeded synthetic activations for the mixed-step workloads.

This module is shared, as a source of inputs only, by both sides of every parity check: the
oracle under ``oracle/`` and the HIP path.  It contains none of the method's arithmetic (no
rotary embedding, no attention, no scheduling).  It only maps a coordinate

    (seed, tensor, request, position, head, dim)   tensor in {q, k, v}

to one number that is approximately standard normal.  The value of a coordinate never depends on
how a prompt is split into chunks, so a chunked run and a monolithic run see identical inputs.

Generator.  The number at a coordinate is the ``counter``-th output of SplitMix64 (Steele, Lea &
Flood, "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014; public-domain reference
code by S. Vigna): with ``gamma = 0x9E3779B97F4A7C15`` the state after ``i + 1`` steps is
``seed + (i + 1) * gamma (mod 2**64)``, and the output is that state passed through the
finaliser (xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31).  The top 16 bits of the
output index a table of 65,536 standard-normal quantiles ``Phi^-1((j + 0.5) / 65536)`` evaluated
in fp64 (``statistics.NormalDist``) and rounded once to fp32; bf16 inputs are that fp32 value
rounded to nearest-even by torch.  All integer work is done in torch int64 with wrap-around, so
the same values come out on the CPU and on a GPU.
"""
from __future__ import annotations

import functools
import statistics

import torch

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

TENSOR_ID = {"q": 0, "k": 1, "v": 2}

# Bit fields of the per-coordinate counter (54 bits in all).
DIM_BITS, HEAD_BITS, POS_BITS, REQ_BITS, TENSOR_BITS = 8, 8, 20, 16, 2
HEAD_SHIFT = DIM_BITS
POS_SHIFT = HEAD_SHIFT + HEAD_BITS
REQ_SHIFT = POS_SHIFT + POS_BITS
TENSOR_SHIFT = REQ_SHIFT + REQ_BITS

TABLE_BITS = 16
TABLE_SIZE = 1 << TABLE_BITS


def _signed(x: int) -> int:
    """The int64 whose two's-complement bits equal the unsigned 64-bit ``x``."""
    x &= MASK64
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns (torch's ``>>`` is arithmetic)."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def splitmix64_at(seed: int, counter: torch.Tensor) -> torch.Tensor:
    """Output number ``counter`` (0-based) of SplitMix64 seeded with ``seed``, as int64 bits."""
    z = (counter + 1) * _signed(GAMMA) + _signed(seed)
    z = (z ^ _lsr(z, 30)) * _signed(MIX1)
    z = (z ^ _lsr(z, 27)) * _signed(MIX2)
    return z ^ _lsr(z, 31)


@functools.lru_cache(maxsize=None)
def _quantile_table_list() -> tuple[float, ...]:
    nd = statistics.NormalDist()
    return tuple(nd.inv_cdf((j + 0.5) / TABLE_SIZE) for j in range(TABLE_SIZE))


@functools.lru_cache(maxsize=None)
def _quantile_table(device: str, dtype: torch.dtype) -> torch.Tensor:
    t32 = torch.tensor(_quantile_table_list(), dtype=torch.float64).to(torch.float32)
    return t32.to(dtype).to(device)


def quantile_table(dtype: torch.dtype = torch.float32, device="cpu") -> torch.Tensor:
    """The 65,536-entry normal-quantile table in ``dtype`` on ``device``."""
    return _quantile_table(str(torch.device(device)), dtype)


def coordinate_counter(tensor: str, req: int, pos: torch.Tensor, n_heads: int, dim: int,
                       head0: int = 0) -> torch.Tensor:
    """Counters for rows ``pos`` (int64 [n]) of one request: int64 [n, n_heads, dim]."""
    if not (0 <= req < (1 << REQ_BITS)):
        raise ValueError(f"request index {req} out of range")
    if n_heads + head0 > (1 << HEAD_BITS) or dim > (1 << DIM_BITS):
        raise ValueError("head or dim out of range")
    dev = pos.device
    base = (TENSOR_ID[tensor] << TENSOR_SHIFT) | (req << REQ_SHIFT)
    heads = (torch.arange(n_heads, dtype=torch.int64, device=dev) + head0) << HEAD_SHIFT
    dims = torch.arange(dim, dtype=torch.int64, device=dev)
    return (base + (pos.to(torch.int64) << POS_SHIFT))[:, None, None] + heads[None, :, None] + dims[None, None, :]


def token_values(seed: int, tensor: str, req: int, pos, n_heads: int, dim: int,
                 dtype: torch.dtype = torch.float32, device="cpu",
                 max_elems: int = 1 << 25) -> torch.Tensor:
    """Values of ``tensor`` for request ``req`` at absolute positions ``pos``.

    Returns ``[len(pos), n_heads, dim]`` in ``dtype`` on ``device``.  ``pos`` may be a
    sequence or an int64 tensor; positions must lie in [0, 2**20).
    """
    pos = torch.as_tensor(pos, dtype=torch.int64, device=device).reshape(-1)
    if pos.numel() and (int(pos.min()) < 0 or int(pos.max()) >= (1 << POS_BITS)):
        raise ValueError("position out of range")
    table = quantile_table(dtype, device)
    out = torch.empty((pos.numel(), n_heads, dim), dtype=dtype, device=device)
    rows = max(1, max_elems // max(1, n_heads * dim))
    for r0 in range(0, pos.numel(), rows):
        ctr = coordinate_counter(tensor, req, pos[r0:r0 + rows], n_heads, dim)
        idx = _lsr(splitmix64_at(seed, ctr), 64 - TABLE_BITS)
        out[r0:r0 + rows] = table[idx]
    return out


def range_values(seed: int, tensor: str, req: int, start: int, stop: int, n_heads: int, dim: int,
                 dtype: torch.dtype = torch.float32, device="cpu") -> torch.Tensor:
    """``token_values`` for the contiguous positions ``[start, stop)``."""
    pos = torch.arange(start, stop, dtype=torch.int64, device=device)
    return token_values(seed, tensor, req, pos, n_heads, dim, dtype=dtype, device=device)


def rows_values(seed: int, tensor: str, reqs, pos, n_heads: int, dim: int,
                dtype: torch.dtype = torch.float32, device="cpu",
                max_elems: int = 1 << 25) -> torch.Tensor:
    """Values of ``tensor`` for rows given by (request, position) pairs: ``[n, n_heads, dim]``.

    Equal to stacking ``token_values(seed, tensor, reqs[i], [pos[i]], ...)`` over the rows.
    """
    reqs = torch.as_tensor(reqs, dtype=torch.int64, device=device).reshape(-1)
    pos = torch.as_tensor(pos, dtype=torch.int64, device=device).reshape(-1)
    if reqs.shape != pos.shape:
        raise ValueError("reqs and pos must have the same length")
    if pos.numel():
        if int(pos.min()) < 0 or int(pos.max()) >= (1 << POS_BITS):
            raise ValueError("position out of range")
        if int(reqs.min()) < 0 or int(reqs.max()) >= (1 << REQ_BITS):
            raise ValueError("request index out of range")
    if n_heads > (1 << HEAD_BITS) or dim > (1 << DIM_BITS):
        raise ValueError("head or dim out of range")
    table = quantile_table(dtype, device)
    out = torch.empty((pos.numel(), n_heads, dim), dtype=dtype, device=device)
    heads = torch.arange(n_heads, dtype=torch.int64, device=device) << HEAD_SHIFT
    dims = torch.arange(dim, dtype=torch.int64, device=device)
    hd = heads[:, None] + dims[None, :]
    rows = max(1, max_elems // max(1, n_heads * dim))
    base = TENSOR_ID[tensor] << TENSOR_SHIFT
    for r0 in range(0, pos.numel(), rows):
        rb = base + (reqs[r0:r0 + rows] << REQ_SHIFT) + (pos[r0:r0 + rows] << POS_SHIFT)
        ctr = rb[:, None, None] + hd[None, :, :]
        out[r0:r0 + rows] = table[_lsr(splitmix64_at(seed, ctr), 64 - TABLE_BITS)]
    return out


# ---- matrices (linear-layer weights and hidden states) -----------------------------------------
# A matrix named ``name`` draws from its own SplitMix64 stream: seed' = seed + MATRIX_SEED[name] *
# gamma, number ``row * cols + col``.  Values are the same normal-quantile table entries, times
# ``scale`` in fp32 (one rounding), then rounded into ``dtype``.
MATRIX_SEED = {"hidden": 101, "w_qkv": 102, "w_o": 103, "attn_out": 104}


def matrix_values(seed: int, name: str, rows: int, cols: int, scale: float = 1.0,
                  dtype: torch.dtype = torch.float32, device="cpu",
                  max_elems: int = 1 << 25) -> torch.Tensor:
    """A ``[rows, cols]`` matrix of approximately N(0, scale**2) values."""
    if rows < 0 or cols < 0:
        raise ValueError("bad shape")
    s = _signed(seed + MATRIX_SEED[name] * GAMMA)
    table = quantile_table(torch.float32, device)
    out = torch.empty((rows, cols), dtype=dtype, device=device)
    step = max(1, max_elems // max(1, cols))
    col = torch.arange(cols, dtype=torch.int64, device=device)
    for r0 in range(0, rows, step):
        r = torch.arange(r0, min(rows, r0 + step), dtype=torch.int64, device=device)
        ctr = r[:, None] * cols + col[None, :]
        v = table[_lsr(splitmix64_at(s, ctr), 64 - TABLE_BITS)]
        out[r0:r0 + step] = (v * torch.tensor(scale, dtype=torch.float32, device=device)).to(dtype)
    return out
