"""GPU parity of cb_linear (through the C ABI) against the oracle's fp64 definition.

Bar: every compared element within oracle.linear.bound (float32 accumulation in any order plus
one rounding to bfloat16) -- a rigorous per-element bound rather than a fixed tolerance.  Small
shapes are compared in full (every tile shape -- 64 x 64 with K splits, the few-rows tiles 64 x 32,
48 and 64 over all of K, 64 x 128, 128 x 192 and 128 x 128 -- with ragged M, K of one and many
stages); the full-size QKV and output projections
of the budget-512 7B-like layer on sampled rows.
"""
import numpy as np
import pytest
import torch

from chunked_prefill_mixed_decode_amd import binding as cb
from oracle import linear as olin
from synth.values import matrix_values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    cb._lib()
    return torch.device("cuda:0")


def _ws(M, N, K, dev):
    n = cb.cb_linear_workspace_bytes(M, N, K)
    return torch.empty(n, dtype=torch.uint8, device=dev) if n else None


def _inputs(M, N, K, dev, seed=11):
    x = matrix_values(seed, "hidden", M, K, dtype=torch.bfloat16, device=dev)
    w = matrix_values(seed, "w_qkv", N, K, scale=K ** -0.5, dtype=torch.bfloat16, device=dev)
    return x, w


def _check(x, w, y, rows=None):
    xs = x.float().cpu().numpy()
    if rows is not None:
        xs = xs[rows]
    ws = w.float().cpu().numpy()
    got = y.float().cpu().numpy()
    if rows is not None:
        got = got[rows]
    ref = olin.linear(xs, ws)
    lim = olin.bound(xs, ws)
    err = np.abs(got - ref)
    bad = np.argwhere(err > lim)
    print(f"  M={x.shape[0]} N={w.shape[0]} K={x.shape[1]}: max|err| {err.max():.3e}, "
          f"max err/bound {float((err / lim).max()):.3f}", flush=True)
    assert not len(bad), f"{len(bad)} elements outside the bound; first {tuple(bad[0])}"


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (37, 256, 192), (130, 384, 64), (300, 128, 1024),
                                   (257, 256, 4096),
                                   (64, 2048, 4096),      # 64 x 64 tiles, K split in eight
                                   (1, 8192, 64), (37, 8192, 1024),   # 64 x 32 tiles over all of K
                                   (50, 12288, 1088),     # 64 x 48 tiles
                                   (9, 16384, 192),       # 64 x 64 tiles over all of K
                                   (500, 12288, 128),     # 128 x 192 tiles, ragged last row tile
                                   (1030, 4096, 128)])    # 128 x 128 tiles, ragged last row tile
def test_linear_small_every_element(dev, M, N, K):
    x, w = _inputs(M, N, K, dev)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    cb.cb_linear(x, w, y, _ws(M, N, K, dev))
    torch.cuda.synchronize()
    _check(x, w, y)


@pytest.mark.parametrize("name,M,N,K", [("qkv, mixed step", 512, 12288, 4096),
                                        ("qkv, decode only", 64, 12288, 4096),
                                        ("output projection, mixed step", 512, 4096, 4096),
                                        ("output projection, decode only", 64, 4096, 4096)])
def test_linear_full_size_sampled_rows(dev, name, M, N, K):
    x, w = _inputs(M, N, K, dev, seed=12)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = _ws(M, N, K, dev)
    cb.cb_linear(x, w, y, ws)
    y2 = torch.empty_like(y)
    cb.cb_linear(x, w, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))          # run-to-run bitwise
    rows = sorted(set(np.random.default_rng(M).choice(M, size=min(M, 12), replace=False).tolist()) | {0, M - 1})
    print(f"[{name}]", flush=True)
    _check(x, w, y, rows)


def test_linear_edge_cases(dev):
    x, w = _inputs(4, 128, 64, dev)
    y = torch.zeros((0, 128), dtype=torch.bfloat16, device=dev)
    cb.cb_linear(x[:0], w, y)                                   # M = 0: nothing to do
    for bad_n, bad_k in ((100, 64), (128, 96)):
        with pytest.raises(cb.CbError) as e:
            cb._check(cb._lib().cb_linear(None, cb.CB_BF16, 4, bad_n, bad_k, cb._ptr(x), cb._ptr(w),
                                          cb._ptr(x), None, 0), "cb_linear")
        assert e.value.status == cb.CB_ERR_INVALID
    with pytest.raises(cb.CbError) as e:                         # float32 is not supported
        cb._check(cb._lib().cb_linear(None, cb.CB_F32, 4, 128, 64, cb._ptr(x), cb._ptr(w), cb._ptr(x),
                                      None, 0), "cb_linear")
    assert e.value.status == cb.CB_ERR_INVALID
    yy = torch.empty((4, 129), dtype=torch.bfloat16, device=dev)
    with pytest.raises(cb.CbError) as e:                         # misaligned output
        cb._check(cb._lib().cb_linear(None, cb.CB_BF16, 4, 128, 64, cb._ptr(x), cb._ptr(w),
                                      yy.data_ptr() + 2, None, 0), "cb_linear")
    assert e.value.status == cb.CB_ERR_INVALID
    # a shape that splits K needs its workspace: too small -> CB_ERR_CAPACITY, nothing launched
    need = cb.cb_linear_workspace_bytes(64, 2048, 4096)
    assert need > 0
    x2, w2 = _inputs(64, 2048, 4096, dev)
    y2 = torch.empty((64, 2048), dtype=torch.bfloat16, device=dev)
    small = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(cb.CbError) as e:
        cb.cb_linear(x2, w2, y2, small)
    assert e.value.status == cb.CB_ERR_CAPACITY
