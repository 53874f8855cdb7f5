"""Rotary position embedding at absolute positions, and bf16 rounding (oracle; test only).

Chunked Prefill 的 Token 预算 (zwjcode), §06 and §07: a chunk's rows carry their absolute positions
(a chunk at offset c starts at position c, never at 0), and the rotary phase is a function of that
absolute position, so a chunked prompt rotates exactly as the unchunked prompt does.

The pages fix neither the rotary variant nor its precision.  Reading used here (parity unpinned by
the pages as to the choice; the arithmetic below is pinned by tests):

* rotate-half layout over the full head dimension D: pair (i, i + D/2) for i < D/2;
* frequency theta_i = base ** (-2 i / D) with base 10000, correctly rounded to fp64;
* table[p, i] = fp32(cos(p * theta_i)), table[p, D/2 + i] = fp32(sin(p * theta_i)): the angle is
  the fp64 product of p and theta_i; its cosine and sine are evaluated in x87 extended precision
  (numpy longdouble) and rounded once to fp32 -- for practical purposes the correctly rounded
  fp32 value of the exact cosine of that fp64 angle (vectorised fp64 libraries lose relative
  accuracy near the zeros of cos and sin, which would change the fp32 rounding there);
* for x in fp32 (bf16 inputs are widened exactly), c = table[p, i], s = table[p, D/2 + i]:
      out[i]       = fp32( fp32(x[i] * c)       - fp32(x[i + D/2] * s) )
      out[i + D/2] = fp32( fp32(x[i + D/2] * c) + fp32(x[i] * s) )
  with every product and sum rounded to fp32 on its own (no fused multiply-add), then the result
  rounded to nearest-even into the storage type.  V is not rotated.

NumPy float32 ufuncs round each operation separately, which is exactly this definition.
"""
from __future__ import annotations

import decimal

import numpy as np


def frequencies(D: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base ** (-2 i / D), correctly rounded to fp64 (50-digit decimal arithmetic)."""
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        b = decimal.Decimal(base)
        return np.array([float(b ** (decimal.Decimal(-2 * i) / decimal.Decimal(D))) for i in range(D // 2)],
                        dtype=np.float64)


def cos_sin_table(max_pos: int, D: int, base: float = 10000.0) -> np.ndarray:
    """[max_pos, D] float32: cos in the first D/2 columns, sin in the last D/2."""
    if D % 2:
        raise ValueError("head dimension must be even")
    if np.finfo(np.longdouble).nmant != 63:
        raise RuntimeError("the table is defined with x87 extended precision (numpy longdouble with a 64-bit significand)")
    theta = frequencies(D, base)
    ang = (np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]).astype(np.longdouble)
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 holding them."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.ascontiguousarray(x, dtype=np.float32))
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = np.where(nan, np.uint64(0x7FC0), r)
    return (r.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(np.shape(x))


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 ``x`` into the storage type ``dtype`` ("f32" or "bf16"), kept as float32."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


def rotate(x: np.ndarray, positions: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rotate float32 rows ``x[..., n, H, D]`` by the angles of ``positions[n]``; float32 out."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    h = D // 2
    t = table[np.asarray(positions)]                    # [n, D]
    c = t[:, None, :h]
    s = t[:, None, h:]
    x1 = x[..., :h]
    x2 = x[..., h:]
    out = np.empty_like(x)
    out[..., :h] = np.subtract(np.multiply(x1, c), np.multiply(x2, s))
    out[..., h:] = np.add(np.multiply(x2, c), np.multiply(x1, s))
    return out


def rotate_stored(x: np.ndarray, positions: np.ndarray, table: np.ndarray, dtype: str) -> np.ndarray:
    """``rotate`` followed by rounding into the storage type."""
    return round_to(rotate(x, positions, table), dtype)
