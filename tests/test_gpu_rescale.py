"""Online softmax under scores that jump: the chunk tiles' lazy rescale and the split merges.

The chunk loop lets its running maximum lag a row's true maximum by up to 8 (base-2 exponent
units) and rescales the output accumulator only when a stage's maximum passes that limit.
Ordinary N(0, 1) inputs move a row's maximum a little in its first stages and rarely after, so
they leave that path nearly idle.  These inputs drive it: every key's vector lies in the head
dimension's lowest-frequency rotary pair (dimension 63 of 128, frequency 10000^(-126/128), so the
rotation turns a key by at most 0.35 rad over these contexts) with a magnitude a(p) that follows a
pattern along the sequence, and every query points the same way, so a row's score for key p is
about a(p) times a constant:

* ``steep``: a(p) = p, the maximum jumps by ~16 per 32-key stage (a rescale at nearly every
  stage, earlier weights decaying to nothing);
* ``gentle``: a(p) = p / 4, jumps of ~4 per stage (weights within the lag limit for a stage or
  two between rescales, so the lag itself matters);
* ``saw``: a(p) = 60 ((p div 100) mod 4), levels that rise past the limit and fall back.

Values are the seeded generator's.  One mixed step (three decodes of up to 3,000 keys and a
600-row chunk after a 2,000-token cached prefix, whose tiles split their keys four ways, so the
combine merges partials of very different maxima), then the chunk rows alone; every row and head
is compared with the oracle's fp64 attention (``oracle.attention.attend`` on the oracle's own
rotation of the same raw inputs) at the bfloat16 bar.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import rope as orope
from synth import values
from synth.workloads import _make
from tests.harness import DeviceRun, TORCH_DTYPE, cached_tokens, compare, plan_of_meta

pytestmark = pytest.mark.gpu

DIM = 63          # first half of the lowest-frequency rotary pair (i = D/2 - 1)
Q_MAG = 4.0


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    from chunked_prefill_mixed_decode_amd import binding
    binding._lib()
    return torch.device("cuda:0")


def magnitude(pattern: str, pos: np.ndarray) -> np.ndarray:
    pos = np.asarray(pos, dtype=np.float64)
    if pattern == "steep":
        return pos
    if pattern == "gentle":
        return pos / 4.0
    if pattern == "saw":
        return 60.0 * ((pos // 100) % 4)
    raise ValueError(pattern)


def raw_keys(pattern: str, pos, Hkv: int, D: int) -> np.ndarray:
    """[n, Hkv, D] float32, rounded to bfloat16: a(p) in dimension DIM, zero elsewhere."""
    k = np.zeros((len(pos), Hkv, D), dtype=np.float32)
    k[:, :, DIM] = magnitude(pattern, pos)[:, None]
    return orope.bf16_round(k)


def raw_queries(n: int, Hq: int, D: int) -> np.ndarray:
    q = np.zeros((n, Hq, D), dtype=np.float32)
    q[:, :, DIM] = Q_MAG
    return q


def workload():
    return _make("rescale_jumps", "bf16", 8, 2, 128, 16, 700, (3000, 900, 37), ((2600, 2000),), 1, 3201,
                 np.random.default_rng(32))


def populate(g: DeviceRun, w, pattern: str):
    bs = w.block_size
    dt = TORCH_DTYPE[w.dtype]
    for rid, n in cached_tokens(w):
        blocks = torch.tensor(g.cb.cb_sched_get_blocks(g.sched, rid), dtype=torch.int64, device=g.device)
        pos = torch.arange(n, dtype=torch.int64, device=g.device)
        slots = (blocks[pos // bs] * bs + pos % bs).to(torch.int32)
        k = torch.from_numpy(raw_keys(pattern, np.arange(n), w.Hkv, w.D)).to(device=g.device, dtype=dt)
        v = values.token_values(w.seed, "v", rid, pos, w.Hkv, w.D, dt, g.device)
        g.runner.append_rows(pos.to(torch.int32), slots, k, v)
        g.written += n


def expected(w, plan, pattern: str) -> dict:
    """Every row: the oracle's rotation of the raw inputs, then its fp64 attention."""
    table = orope.cos_sin_table(w.max_position(), w.D)
    cu = plan["cu_seqlens_q"]
    out = {}
    for s in range(plan["num_seqs"]):
        rows = list(range(cu[s], cu[s + 1]))
        rid = plan["seq_ids"][s]
        pos = np.array([plan["positions"][r] for r in rows])
        P = int(pos.max()) + 1
        kpos = np.arange(P)
        kh = orope.rotate_stored(raw_keys(pattern, kpos, w.Hkv, w.D), kpos, table, w.dtype)
        v = values.token_values(w.seed, "v", rid, torch.as_tensor(kpos), w.Hkv, w.D,
                                TORCH_DTYPE[w.dtype], "cpu").float().numpy()
        qh = orope.rotate_stored(raw_queries(len(rows), w.Hq, w.D), pos, table, w.dtype)
        res = oattn.attend(qh, kh, v, pos, w.D ** -0.5)
        for i, r in enumerate(rows):
            out[r] = res[i]
    return out


def check(out, want, rows, tag):
    rs = sorted(rows)
    ok, mabs, mrel = compare(out.float().cpu().numpy()[rs], np.stack([want[r] for r in rs]), "bf16")
    say(f"  {tag}: {len(rs)} rows, max|err| {mabs:.3e}, max rel {mrel:.3e}")
    assert ok, f"{tag}: max abs {mabs}, max rel {mrel}"


@pytest.mark.parametrize("pattern", ["steep", "gentle", "saw"])
def test_jumping_scores(dev, pattern):
    w = workload()
    g = DeviceRun(w, dev, populate=False)
    populate(g, w, pattern)
    cb = g.cb
    meta = g.runner.build(g.sched, w.budget)
    dm = g.runner.upload(meta)
    plan = plan_of_meta(meta)
    T, nd = meta.num_tokens, meta.num_decodes
    h = meta.host
    dt = TORCH_DTYPE[w.dtype]
    pos = h["positions"][:T].numpy()
    q = torch.from_numpy(raw_queries(T, w.Hq, w.D)).to(device=dev, dtype=dt)
    k = torch.from_numpy(raw_keys(pattern, pos, w.Hkv, w.D)).to(device=dev, dtype=dt)
    qlens = (h["cu_seqlens_q"][1:meta.num_seqs + 1] - h["cu_seqlens_q"][:meta.num_seqs]).long()
    reqs = torch.repeat_interleave(h["seq_ids"][:meta.num_seqs].long(), qlens).to(dev)
    v = values.rows_values(w.seed, "v", reqs, torch.as_tensor(pos, dtype=torch.int64, device=dev), w.Hkv, w.D,
                           dt, dev)
    q_rot, out = torch.empty_like(q), torch.empty_like(q)
    g.runner.append(dm, q, k, v, q_rot)
    g.runner.attend(meta, dm, q_rot, out)
    torch.cuda.synchronize()
    say(f"[{pattern}] T={T} nd={nd}")
    want = expected(w, plan, pattern)
    check(out, want, set(range(T)), f"{pattern} mixed")
    # The chunk rows alone (a chunk-only launch plans its own key split).
    cu_chunk = (dm["cu_seqlens_q"][nd:meta.num_seqs + 1] - nd).contiguous()
    chunk_ctx = int(h["context_lens"][nd:meta.num_seqs].max())
    g.runner.ensure_workspace(cb.cb_attn_workspace_bytes(meta.num_seqs - nd, 0, T - nd, meta.max_q_len, 0,
                                                         chunk_ctx, w.Hq, w.Hkv, w.D))
    out_c = torch.empty_like(out[nd:])
    cb.cb_mixed_paged_attention(q_rot[nd:], g.runner.k_cache, g.runner.v_cache, cu_chunk,
                                dm["context_lens"][nd:], dm["cu_blocks"][nd:], dm["block_table"], out_c,
                                g.runner.workspace, num_seqs=meta.num_seqs - nd, num_decodes=0,
                                max_q_len=meta.max_q_len, max_decode_ctx=0, max_ctx=chunk_ctx,
                                scale=g.runner.scale)
    torch.cuda.synchronize()
    check(torch.cat([out[:nd], out_c]), want, set(range(nd, T)), f"{pattern} chunk-only")
