"""Launches of chunk rows alone (no decode rows) against the oracle.

A launch without decode rows plans its own key split (at least 512 keys per split, up to 512
tiles), so its tiles and its combine differ from those of the mixed launch the same rows take
part in.  Each step of a workload runs as usual; then the step's chunk rows are launched alone
(the cache holds every key they see by then) and compared with the oracle's fp64 attention of the
same rows: every chunk row of the scaled-down bfloat16 workloads (GQA groups, head dim 64, several
chunks per launch, prefill-only steps), at the budget-512 layer every step (128 to 512 tiles,
unsplit, two-, four- and eight-way splits), and a 1024-row GQA-8 chunk whose launch takes 256
unsplit 8-wave tiles of 256 rows, these two on the first 64, the last 64 and 128 seeded random
chunk rows.
"""
import numpy as np
import pytest
import torch

from synth import workloads
from tests.harness import DeviceRun, OracleRun, compare

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    from chunked_prefill_mixed_decode_amd import binding
    binding._lib()
    return torch.device("cuda:0")


def run_step(g: DeviceRun):
    """One ordinary step (arrivals, build, pull, rope + append, attention); returns the step's
    metadata, its device views and the rotated queries."""
    g.arrive(g.step_index)
    g.step_index += 1
    meta = g.runner.build(g.sched, g.w.budget)
    dm = g.runner.upload(meta)
    q, k, v = g.step_inputs(meta)
    q_rot, out = torch.empty_like(q), torch.empty_like(q)
    g.runner.append(dm, q, k, v, q_rot)
    g.runner.attend(meta, dm, q_rot, out)
    g.written += meta.num_tokens
    return meta, dm, q_rot


def chunk_only(g: DeviceRun, meta, dm, q_rot):
    """The step's chunk rows launched alone: [T - nd, Hq, D]."""
    w, cb = g.w, g.cb
    nd, T, S = meta.num_decodes, meta.num_tokens, meta.num_seqs
    ctx = int(meta.host["context_lens"][nd:S].max())
    cu = (dm["cu_seqlens_q"][nd:S + 1] - nd).contiguous()
    g.runner.ensure_workspace(cb.cb_attn_workspace_bytes(S - nd, 0, T - nd, meta.max_q_len, 0, ctx,
                                                         w.Hq, w.Hkv, w.D))
    out = torch.empty_like(q_rot[nd:])
    cb.cb_mixed_paged_attention(q_rot[nd:], g.runner.k_cache, g.runner.v_cache, cu, dm["context_lens"][nd:],
                                dm["cu_blocks"][nd:], dm["block_table"], out, g.runner.workspace,
                                num_seqs=S - nd, num_decodes=0, max_q_len=meta.max_q_len, max_decode_ctx=0,
                                max_ctx=ctx, scale=g.runner.scale)
    torch.cuda.synchronize()
    return out


def tiles_of(w, meta) -> int:
    """Query tiles of the launch before key splits (128 rows: positions x heads of a group)."""
    G = w.Hq // w.Hkv
    bmq = max(1, 128 // G)
    return sum(w.Hkv * -(-(meta.host["cu_seqlens_q"][s + 1] - meta.host["cu_seqlens_q"][s]).item() // bmq)
               for s in range(meta.num_decodes, meta.num_seqs))


def check(ora: OracleRun, plan, out_c, nd: int, rows, tag: str, dtype: str):
    want = ora.expected_rows(plan, rows)
    rs = sorted(want)
    got = out_c.float().cpu().numpy()[[r - nd for r in rs]]
    ok, mabs, mrel = compare(got, np.stack([want[r] for r in rs]), dtype)
    say(f"  {tag}: {len(rs)} chunk rows, max|err| {mabs:.3e}, max rel {mrel:.3e}")
    assert ok, f"{tag}: max abs {mabs}, max rel {mrel}"


@pytest.mark.parametrize("i", [i for i in workloads.SMALL if workloads.small(i).dtype == "bf16"])
def test_small_chunk_rows_alone(dev, i):
    w = workloads.small(i)
    g = DeviceRun(w, dev)
    ora = OracleRun(w, value_device=dev)
    step = 0
    while (w.steps is None and ora.b.pending_prompts() > 0) or (w.steps is not None and step < w.steps):
        plan = ora.build()
        meta, dm, q_rot = run_step(g)
        nd, T = meta.num_decodes, meta.num_tokens
        if T > nd:
            out_c = chunk_only(g, meta, dm, q_rot)
            check(ora, plan, out_c, nd, range(nd, T), f"[{w.name}] step {step} ({tiles_of(w, meta)} tiles)",
                  w.dtype)
        step += 1


def sampled_rows(nd: int, T: int, seed: int):
    """The first 64, the last 64 and 128 seeded random chunk rows."""
    rng = np.random.default_rng(seed)
    chunk = np.arange(nd, T)
    rows = set(chunk[:64].tolist()) | set(chunk[-64:].tolist())
    rest = chunk[64:-64]
    if len(rest):
        rows |= set(rng.choice(rest, size=min(128, len(rest)), replace=False).tolist())
    return rows


def test_budget512_chunk_rows_alone(dev):
    w = workloads.get(2)
    g = DeviceRun(w, dev)
    ora = OracleRun(w, value_device=dev)
    for step in range(w.steps):
        plan = ora.build()
        meta, dm, q_rot = run_step(g)
        nd, T = meta.num_decodes, meta.num_tokens
        out_c = chunk_only(g, meta, dm, q_rot)
        check(ora, plan, out_c, nd, sampled_rows(nd, T, 100 + step),
              f"[{w.name}] step {step} ({tiles_of(w, meta)} tiles)", w.dtype)


@pytest.mark.parametrize("bs", [8, 32, 256])
def test_wide_tiles_chunk_rows_alone(dev, bs):
    """64 query / 8 KV heads, head dim 128, blocks of 8, 32 or 256 tokens: two decodes and a
    1024-row chunk after 256 cached tokens.  Launched alone, the chunk fills 32 x 8 = 256 tiles of
    256 rows (32 positions x 8 heads) without a key split, which a 256-compute-unit device runs as
    8-wave tiles (each wave copies 4 key rows of a stage, inside one block of any size)."""
    rng = np.random.Generator(np.random.PCG64(2010))
    ctx = rng.integers(100, 600, size=2, endpoint=True)
    w = workloads._make(f"wide_gqa8_chunk1024_bs{bs}_bf16", "bf16", 64, 8, 128, bs, 1026, ctx, ((1280, 256),), 1,
                        2010, rng)
    g = DeviceRun(w, dev)
    ora = OracleRun(w, value_device=dev)
    plan = ora.build()
    meta, dm, q_rot = run_step(g)
    nd, T = meta.num_decodes, meta.num_tokens
    assert T - nd == 1024
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    say(f"  256-row tiles: {-(-1024 // 32) * 8}, compute units: {cus}")
    out_c = chunk_only(g, meta, dm, q_rot)
    check(ora, plan, out_c, nd, sampled_rows(nd, T, 110), f"[{w.name}] (256 unsplit 256-row tiles)", w.dtype)
