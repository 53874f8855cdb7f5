"""GPU parity of the HIP path (through the C ABI) against the oracle.

Bars: step metadata and every written K/V slot bit-exact; rotated queries bit-exact; attention
outputs |gpu - oracle| <= atol + rtol |oracle| with (atol, rtol) = (1e-4, 0) for float32 and
(2e-2, 1e-2) for bfloat16 (float32 accumulation).  Cache elements outside the written slots keep
their all-ones sentinel.  Scaled-down workloads are checked on every row of every step; the five
full-size workloads on sampled rows and slots, in the same launch configuration as the benchmark.
"""
import numpy as np
import pytest
import torch

from oracle import attention as oattn
from oracle import rope as orope
from synth import workloads
from tests.harness import DeviceRun, OracleRun, bits_of, cached_tokens, compare, plan_of_meta

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    from chunked_prefill_mixed_decode_amd import binding
    binding._lib()
    return torch.device("cuda:0")


def check_metadata(meta, plan):
    got = plan_of_meta(meta)
    for k in ("seq_ids", "cu_seqlens_q", "context_lens", "cu_blocks", "block_table", "positions",
              "slot_mapping", "num_seqs", "num_decodes", "num_tokens", "unused_tokens"):
        assert got[k] == plan[k], k


def check_step_kv(gpu: DeviceRun, ora: OracleRun, plan, rows):
    """K/V written by the step's ``rows`` are bit-exact."""
    cu = plan["cu_seqlens_q"]
    for s in range(plan["num_seqs"]):
        srows = [r for r in range(cu[s], cu[s + 1]) if r in rows]
        if not srows:
            continue
        rid = plan["seq_ids"][s]
        pos = np.array([plan["positions"][r] for r in srows])
        slots = np.array([plan["slot_mapping"][r] for r in srows])
        kw, vw = ora.expected_kv(rid, pos)
        _, _, kb, vb = gpu.cache_rows(slots)
        for name, got, want in (("K", kb, bits_of(kw, gpu.w.dtype)), ("V", vb, bits_of(vw, gpu.w.dtype))):
            bad = np.argwhere(got != want)
            if len(bad):
                i = tuple(bad[0])
                say(f"  {name} mismatch request {rid}: {len(bad)} of {got.size} elements; first at "
                    f"(row {i[0]} pos {pos[i[0]]}, head {i[1]}, dim {i[2]}): got {got[i]} want {want[i]}")
            assert not len(bad), f"{name} slots of request {rid}"


def check_kv_rows(gpu: DeviceRun, ora: OracleRun, reqs, pos, slots, tag):
    """K and V at ``slots`` equal the oracle's rotated keys and raw values of (reqs, pos), bit for
    bit ("Chunked Prefill 的 Token 预算" §06: slot_mapping names where each token's K/V lands)."""
    kw, vw = ora.expected_kv_rows(reqs, pos)
    _, _, kb, vb = gpu.cache_rows(np.asarray(slots))
    for name, got, want in (("K", kb, bits_of(kw, gpu.w.dtype)), ("V", vb, bits_of(vw, gpu.w.dtype))):
        bad = np.argwhere(got != want)
        if len(bad):
            i = tuple(bad[0])
            say(f"  {tag}: {name} mismatch at {len(bad)} of {got.size} elements; first at request "
                f"{reqs[i[0]]} pos {pos[i[0]]}, head {i[1]}, dim {i[2]}: got {got[i]} want {want[i]}")
        assert not len(bad), f"{tag}: {name} slots"


def check_step_kv_all(gpu: DeviceRun, ora: OracleRun, plan, tag):
    """Every slot the step wrote (all its rows) is bit-exact."""
    T = plan["num_tokens"]
    if T == 0:
        return
    cu = plan["cu_seqlens_q"]
    reqs = np.repeat(np.array(plan["seq_ids"][:plan["num_seqs"]]), np.diff(np.array(cu[:plan["num_seqs"] + 1])))
    check_kv_rows(gpu, ora, reqs, np.array(plan["positions"][:T]), np.array(plan["slot_mapping"][:T]), tag)


def check_setup_sample(gpu: DeviceRun, ora: OracleRun, w, frac: float, seed: int):
    """A seeded sample (at least ``frac`` of them, and the first and last of each request) of the
    slots written at set-up (the cached contexts) is bit-exact."""
    rng = np.random.default_rng(seed)
    reqs, pos, slots = [], [], []
    for rid, n in cached_tokens(w):
        blocks = np.array(gpu.cb.cb_sched_get_blocks(gpu.sched, rid))
        take = max(2, int(np.ceil(frac * n)))
        p = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, take), replace=False)]))
        reqs.append(np.full(len(p), rid))
        pos.append(p)
        slots.append(blocks[p // w.block_size] * w.block_size + p % w.block_size)
    reqs, pos, slots = np.concatenate(reqs), np.concatenate(pos), np.concatenate(slots)
    say(f"  set-up sample: {len(pos)} slots")
    for a in range(0, len(pos), 1 << 16):
        b = min(len(pos), a + (1 << 16))
        check_kv_rows(gpu, ora, reqs[a:b], pos[a:b], slots[a:b], "set-up")


def check_q_rot(gpu: DeviceRun, ora: OracleRun, plan, q_rot, rows):
    cu = plan["cu_seqlens_q"]
    got = q_rot.float().cpu().numpy()
    for s in range(plan["num_seqs"]):
        srows = [r for r in range(cu[s], cu[s + 1]) if r in rows]
        if not srows:
            continue
        pos = np.array([plan["positions"][r] for r in srows])
        want = orope.rotate_stored(ora.raw("q", plan["seq_ids"][s], pos), pos, ora.table, gpu.w.dtype)
        assert np.array_equal(bits_of(got[srows], gpu.w.dtype), bits_of(want, gpu.w.dtype))


def check_outputs(gpu: DeviceRun, ora: OracleRun, plan, out, rows, tag):
    want = ora.expected_rows(plan, rows)
    got = out.float().cpu().numpy()
    rs = sorted(want)
    ok, mabs, mrel = compare(got[rs], np.stack([want[r] for r in rs]), gpu.w.dtype)
    say(f"  {tag}: {len(rs)} rows, max|err| {mabs:.3e}, max rel {mrel:.3e}")
    assert ok, f"{tag}: max abs {mabs}, max rel {mrel}"
    return mabs


def sample_rows(plan, n_dec, n_chunk, seed):
    rng = np.random.default_rng(seed)
    nd, T = plan["num_decodes"], plan["num_tokens"]
    rows = set()
    if nd:
        rows |= set(rng.choice(nd, size=min(n_dec, nd), replace=False).tolist())
        rows |= {0, nd - 1}
    if T > nd:
        cu = plan["cu_seqlens_q"]
        for s in range(nd, plan["num_seqs"]):                 # first and last rows of each chunk
            rows |= {cu[s], cu[s + 1] - 1}
        rows |= set((nd + rng.choice(T - nd, size=min(n_chunk, T - nd), replace=False)).tolist())
    return rows


# ---------------------------------------------------------------------------------------------
# Scaled-down workloads: every row of every step.
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("i", workloads.SMALL)
def test_small_workload_every_row_every_step(dev, i):
    w = workloads.small(i)
    say(f"[{w.name}] set-up")
    gpu = DeviceRun(w, dev)
    ora = OracleRun(w, value_device=dev)
    step = 0
    while (w.steps is None and ora.b.pending_prompts() > 0) or (w.steps is not None and step < w.steps):
        say(f"[{w.name}] step {step}")
        plan = ora.build()
        meta, out, q_rot = gpu.step()
        torch.cuda.synchronize()
        check_metadata(meta, plan)
        rows = set(range(plan["num_tokens"]))
        check_step_kv(gpu, ora, plan, rows)
        check_q_rot(gpu, ora, plan, q_rot, rows)
        check_outputs(gpu, ora, plan, out, None, f"step {step}")
        step += 1
        assert step <= w.max_steps
    # set-up slots too, and nothing written outside the slots
    nd = len(w.decode_ctx)
    for rid, n in [(r, c) for r, c in enumerate(w.decode_ctx)] + \
                  [(nd + j, c) for j, (_, c) in enumerate(w.prompts) if c]:
        blocks = np.array(gpu.cb.cb_sched_get_blocks(gpu.sched, rid))
        pos = np.arange(n)
        slots = blocks[pos // w.block_size] * w.block_size + pos % w.block_size
        kw, vw = ora.expected_kv(rid, pos)
        _, _, kb, vb = gpu.cache_rows(slots)
        assert np.array_equal(kb, bits_of(kw, w.dtype)) and np.array_equal(vb, bits_of(vw, w.dtype))
    total = 2 * gpu.runner.k_cache.numel()
    assert gpu.sentinel_count() == total - 2 * gpu.written * w.Hkv * w.D


# ---------------------------------------------------------------------------------------------
# Full-size workloads: sampled rows and slots at the benchmark's launch configuration.
# ---------------------------------------------------------------------------------------------
FULL_SAMPLE = {1: (8, 8, 1), 2: (8, 24, 1), 3: (8, 24, 1), 4: (4, 12, 1), 5: (None, None, 1)}


def stratified_rows(plan, seed):
    """All decode rows; of the chunk rows the first 64, the last 64 and 128 seeded random others."""
    rng = np.random.default_rng(seed)
    nd, T = plan["num_decodes"], plan["num_tokens"]
    chunk = np.arange(nd, T)
    rows = set(range(nd)) | set(chunk[:64].tolist()) | set(chunk[-64:].tolist())
    rest = chunk[64:-64]
    if len(rest):
        rows |= set(rng.choice(rest, size=min(128, len(rest)), replace=False).tolist())
    return rows


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_workload_sampled(dev, cfg):
    w = workloads.get(cfg)
    n_dec, n_chunk, every = FULL_SAMPLE[cfg]
    say(f"[{w.name}] set-up: {len(w.decode_ctx)} decodes, {w.num_blocks} blocks")
    gpu = DeviceRun(w, dev)
    ora = OracleRun(w, value_device=dev)
    check_setup_sample(gpu, ora, w, 0.01, seed=cfg)
    step = 0
    while (w.steps is None and ora.b.pending_prompts() > 0) or (w.steps is not None and step < w.steps):
        plan = ora.build()
        meta, out, q_rot = gpu.step()
        torch.cuda.synchronize()
        check_metadata(meta, plan)
        check_step_kv_all(gpu, ora, plan, f"step {step}")
        if step % every == 0 or step == (w.steps or 0) - 1:
            say(f"[{w.name}] step {step}: T={plan['num_tokens']} nd={plan['num_decodes']}")
            rows = stratified_rows(plan, seed=step) if n_dec is None else sample_rows(plan, n_dec, n_chunk, seed=step)
            check_q_rot(gpu, ora, plan, q_rot, rows)
            check_outputs(gpu, ora, plan, out, rows, f"step {step}")
        step += 1
    total = 2 * gpu.runner.k_cache.numel()
    assert gpu.sentinel_count() == total - 2 * gpu.written * w.Hkv * w.D


# ---------------------------------------------------------------------------------------------
# Invariants of the method on the GPU path.
# ---------------------------------------------------------------------------------------------
def test_chunked_run_equals_monolithic_run(dev):
    # "Chunked Prefill 的 Token 预算", intro and §02: chunking changes when work happens, not the
    # final cache; rows match the unchunked computation.
    w = workloads.small(2)
    big = w.budget * 8
    chunked, mono = DeviceRun(w, dev), DeviceRun(w, dev, max_budget=big)
    prompt = len(w.decode_ctx)
    outs_c, outs_m = {}, {}
    while True:
        meta, out, _ = chunked.step()
        h = plan_of_meta(meta)
        for s in range(meta.num_decodes, meta.num_seqs):
            for r in range(h["cu_seqlens_q"][s], h["cu_seqlens_q"][s + 1]):
                outs_c[h["positions"][r]] = out[r].float().cpu().numpy()
        if gpu_pending(chunked) == 0:
            break
    meta, out, _ = mono.step(budget=big)
    h = plan_of_meta(meta)
    assert meta.num_seqs == len(w.decode_ctx) + 1
    s = meta.num_seqs - 1
    for r in range(h["cu_seqlens_q"][s], h["cu_seqlens_q"][s + 1]):
        outs_m[h["positions"][r]] = out[r].float().cpu().numpy()
    assert sorted(outs_c) == sorted(outs_m) == list(range(w.prompts[0][0]))
    diff = max(float(np.abs(outs_c[p] - outs_m[p]).max()) for p in outs_c)
    say(f"  chunked vs monolithic max|diff| {diff:.3e}")
    assert diff <= 2 * 2e-2
    blocks = np.array(chunked.cb.cb_sched_get_blocks(chunked.sched, prompt))
    assert blocks.tolist() == mono.cb.cb_sched_get_blocks(mono.sched, prompt)
    pos = np.arange(w.prompts[0][0])
    slots = blocks[pos // w.block_size] * w.block_size + pos % w.block_size
    a, b = chunked.cache_rows(slots), mono.cache_rows(slots)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3], b[3])     # bit-identical K and V


def gpu_pending(g: DeviceRun) -> int:
    return g.cb.cb_sched_pending_prompts(g.sched)


def test_run_to_run_bitwise_determinism_and_decode_isolation(dev):
    w = workloads.small(4)
    g = DeviceRun(w, dev)
    g.step()                                   # advance once so chunks have a cached prefix
    snap = g.cb.cb_sched_clone(g.sched)
    meta, out1, _ = g.step()
    out1 = out1.clone()
    g.sched = g.cb.cb_sched_clone(snap)        # replay the same step: identical appends
    meta2, out2, _ = g.step()
    assert meta.num_tokens == meta2.num_tokens and meta.num_prefill_tokens > 0
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    g.sched = g.cb.cb_sched_clone(snap)        # decodes alone: same decode rows, bit for bit
    meta3, out3, _ = g.step(budget=meta.num_decodes)
    assert meta3.num_prefill_tokens == 0
    nd = meta.num_decodes
    assert torch.equal(out1[:nd].view(torch.int16), out3[:nd].view(torch.int16))


def test_planted_mistakes_are_caught(dev):
    # zwjcode §07: a chunk's positions restarted at 0, or its rows blind to the cached prefix,
    # give different results; planted in the oracle, they must fail the parity bar.
    w = workloads.small(3)
    gpu, ora = DeviceRun(w, dev), OracleRun(w, value_device=dev)
    for _ in range(2):
        plan = ora.build()
        meta, out, _ = gpu.step()
    torch.cuda.synchronize()
    nd = plan["num_decodes"]
    s = nd
    cu = plan["cu_seqlens_q"]
    rows = list(range(cu[s], cu[s + 1]))
    pos = np.array([plan["positions"][r] for r in rows])
    c = int(pos[0])
    assert c > 0
    rid = plan["seq_ids"][s]
    got = out[rows].float().cpu().numpy()
    good = np.stack([ora.expected_rows(plan, rows)[r] for r in rows])
    assert compare(got, good, w.dtype)[0]
    # (a) positions reset to 0 inside the chunk
    local = pos - c
    q_bad = orope.rotate_stored(ora.raw("q", rid, pos), local, ora.table, w.dtype)
    kpos = np.arange(pos[-1] + 1)
    kpos_bad = np.concatenate([kpos[:c], kpos[c:] - c])
    k_bad = orope.rotate_stored(ora.raw("k", rid, kpos), kpos_bad, ora.table, w.dtype)
    v = ora.raw("v", rid, kpos)
    bad_a = oattn.attend(q_bad, k_bad, v, pos, ora.scale)
    assert not compare(got, bad_a, w.dtype)[0]
    # (b) chunk-local visibility {c .. c + i}
    kh, _ = ora.expected_kv(rid, kpos)
    qh = orope.rotate_stored(ora.raw("q", rid, pos), pos, ora.table, w.dtype)
    bad_b = oattn.attend(qh, kh[c:], v[c:], pos - c, ora.scale)
    assert not compare(got, bad_b, w.dtype)[0]


def test_edge_steps(dev):
    """Decode-only steps, chunk-only steps, one-token prompts and a one-token budget."""
    from synth.workloads import _make
    rng = np.random.default_rng(0)
    cases = [
        _make("edge_decode_only", "bf16", 4, 2, 128, 16, 3, (17, 1, 64), (), 3, 3001, np.random.default_rng(1)),
        _make("edge_chunk_only", "bf16", 8, 8, 128, 16, 97, (), ((300, 0), (1, 0), (2, 0)), 5, 3002, np.random.default_rng(2)),
        _make("edge_budget_one", "bf16", 2, 1, 64, 8, 1, (), ((5, 0),), 6, 3003, np.random.default_rng(3)),
        _make("edge_cached_all_but_one", "bf16", 4, 4, 128, 32, 64, (40,), ((200, 199),), 2, 3004, np.random.default_rng(4)),
    ]
    del rng
    for w in cases:
        say(f"[{w.name}]")
        gpu, ora = DeviceRun(w, dev), OracleRun(w, value_device=dev)
        for step in range(w.steps):
            plan = ora.build()
            meta, out, q_rot = gpu.step()
            torch.cuda.synchronize()
            check_metadata(meta, plan)
            if plan["num_tokens"] == 0:
                continue
            rows = set(range(plan["num_tokens"]))
            check_step_kv(gpu, ora, plan, rows)
            check_outputs(gpu, ora, plan, out, None, f"{w.name} step {step}")


def test_block_sizes_and_group_widths(dev):
    """Cache blocks of 32, 64 and 256 tokens (a 32-key chunk stage lies inside one block, the block
    address is shared by many stages, partial blocks at both ends of a context), a 24-head group
    (two 16-head blocks per KV head, the second one ragged), 16- and 32-head groups (whole blocks),
    a 128-head group (eight blocks per KV head; a chunk tile holds one position), cache blocks of
    128 tokens, and a chunk-only step whose keys are split the maximum 8 ways; every row of every
    step."""
    from synth.workloads import _make
    cases = [
        _make("edge_bs64_gqa4", "bf16", 8, 2, 128, 64, 200, (300, 1, 129, 700), ((500, 0), (70, 0)), 4, 3011,
              np.random.default_rng(11)),
        _make("edge_bs256_mha", "bf16", 4, 4, 128, 256, 300, (1000, 256, 257), ((600, 100),), 3, 3012,
              np.random.default_rng(12)),
        _make("edge_group24", "bf16", 48, 2, 128, 16, 160, (90, 500, 33), ((300, 0),), 3, 3013,
              np.random.default_rng(13)),
        _make("edge_d64_bs32", "bf16", 8, 8, 64, 32, 100, (64, 65), ((150, 0),), 3, 3014,
              np.random.default_rng(14)),
        # the widest group a chunk tile holds: 128 query heads on one KV head, one position a tile
        _make("edge_group128", "bf16", 128, 1, 64, 16, 40, (70, 3), ((50, 0),), 2, 3015,
              np.random.default_rng(15)),        # exactly one and exactly two 16-head blocks per KV head; cache blocks of 128 tokens
        _make("edge_group16", "bf16", 32, 2, 128, 16, 120, (200, 17), ((150, 0),), 2, 3016,
              np.random.default_rng(16)),
        _make("edge_group32_bs128", "bf16", 64, 2, 64, 128, 120, (300, 129), ((260, 0),), 3, 3017,
              np.random.default_rng(17)),
        # a 20-token chunk after 8200 cached tokens, no decodes: two tiles, keys split 8 ways
        _make("edge_split8", "bf16", 2, 2, 128, 16, 20, (), ((8220, 8200),), 1, 3018,
              np.random.default_rng(18)),
    ]
    for w in cases:
        say(f"[{w.name}]")
        gpu, ora = DeviceRun(w, dev), OracleRun(w, value_device=dev)
        for step in range(w.steps):
            plan = ora.build()
            meta, out, q_rot = gpu.step()
            torch.cuda.synchronize()
            check_metadata(meta, plan)
            if plan["num_tokens"] == 0:
                continue
            check_step_kv(gpu, ora, plan, set(range(plan["num_tokens"])))
            check_outputs(gpu, ora, plan, out, None, f"{w.name} step {step}")


def test_rope_append_skips_invalid_rows(dev):
    from chunked_prefill_mixed_decode_amd.runner import MixedStepRunner
    r = MixedStepRunner(Hq=4, Hkv=2, D=128, block_size=16, num_blocks=4, dtype=torch.bfloat16,
                        device=dev, max_pos=100, cap_seqs=4, cap_tokens=8, cap_blocks=8)
    T = 5
    q = torch.randn(T, 4, 128, device=dev).to(torch.bfloat16)
    k = torch.randn(T, 2, 128, device=dev).to(torch.bfloat16)
    v = torch.randn(T, 2, 128, device=dev).to(torch.bfloat16)
    pos = torch.tensor([3, 100, 7, -1, 9], dtype=torch.int32, device=dev)      # rows 1, 3 invalid
    slots = torch.tensor([0, 1, -1, 3, 64], dtype=torch.int32, device=dev)     # row 2 no slot, row 4 out of range
    q_out = torch.full_like(q, float("nan"))
    r.append({"positions": pos, "slot_mapping": slots}, q, k, v, q_out)
    torch.cuda.synchronize()
    assert torch.isnan(q_out[1].float()).all() and torch.isnan(q_out[3].float()).all()
    assert not torch.isnan(q_out[[0, 2, 4]].float()).any()
    kb = r.k_cache.view(torch.int16)
    written = (kb != -1).any(dim=-1)            # [nb, Hkv, bs]
    assert written.sum().item() == 2            # only row 0 (slot 0), one entry per KV head
    assert written[0, :, 0].all()


def test_host_copy_sees_every_rewrite(dev):
    """cb_copy_host_to_device: the kernel copy reproduces the pinned bytes exactly, also after the
    host rewrites the same buffer (no stale GPU-cached host data), and rejects misalignment."""
    from chunked_prefill_mixed_decode_amd import binding as cb
    g = torch.Generator().manual_seed(7)
    src = torch.empty(12345 * 2, dtype=torch.int32).pin_memory()
    dst = torch.empty(src.numel(), dtype=torch.int32, device=dev)
    for rnd in range(3):
        src.copy_(torch.randint(-2**31, 2**31 - 1, (src.numel(),), generator=g, dtype=torch.int64).to(torch.int32))
        cb.cb_copy_host_to_device(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(dst.cpu(), src), f"round {rnd}"
    lib = cb._lib()
    assert lib.cb_copy_host_to_device(None, src.data_ptr() + 4, dst.data_ptr(), 8) == cb.CB_ERR_INVALID
    assert lib.cb_copy_host_to_device(None, src.data_ptr(), dst.data_ptr(), 12) == cb.CB_ERR_INVALID


@pytest.mark.parametrize("case", ["small4", "small8", "budget512"])
def test_host_decode_plan_matches_device_split(dev, case):
    # The runner ships a host-made decode plan (cb_decode_plan); the same call without it splits on
    # the device.  Same rule, so the outputs must agree bit for bit; a plan made for another wave
    # count is refused.  The budget-512 layer (64 decodes beside a 448-row chunk) puts a chunk tile
    # beside half of the decode workgroups, whose shares the rule lowers.
    w = workloads.get(2) if case == "budget512" else workloads.small(int(case[-1]))
    g = DeviceRun(w, dev)
    cb = g.cb
    for _ in range(2):
        meta = g.runner.build(g.sched, w.budget)
        dm = g.runner.upload(meta)
        q, k, v = g.step_inputs(meta)
        q_rot, out_plan, out_dev = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        g.runner.append(dm, q, k, v, q_rot)
        g.runner.attend(meta, dm, q_rot, out_plan)
        assert meta.plan_waves > 0
        kw = dict(num_seqs=meta.num_seqs, num_decodes=meta.num_decodes, max_q_len=meta.max_q_len,
                  max_decode_ctx=meta.max_decode_context_len, max_ctx=meta.max_context_len,
                  scale=g.runner.scale)
        cb.cb_mixed_paged_attention(q_rot, g.runner.k_cache, g.runner.v_cache, dm["cu_seqlens_q"],
                                    dm["context_lens"], dm["cu_blocks"], dm["block_table"], out_dev,
                                    g.runner.workspace, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out_plan.view(torch.int16), out_dev.view(torch.int16))
        with pytest.raises(cb.CbError) as e:
            cb.cb_mixed_paged_attention(q_rot, g.runner.k_cache, g.runner.v_cache, dm["cu_seqlens_q"],
                                        dm["context_lens"], dm["cu_blocks"], dm["block_table"], out_dev,
                                        g.runner.workspace, decode_plan=dm["decode_plan"],
                                        plan_waves=meta.plan_waves + 4, **kw)
        assert e.value.status == cb.CB_ERR_INVALID


# ---------------------------------------------------------------------------------------------
# Builder policies and caps other than the default, through the kernels.
# ---------------------------------------------------------------------------------------------
POLICY_CASES = [
    # "Splitting Prefill From Decode Inside a Step", "Choosing the priority order": prefill-first
    # gives the prompts the whole budget; the decodes run only in what is left (here: not until
    # the prompts are through, then all of them).
    ("prefill_first", dict(policy=1), (900, 40, 2000, 333, 17), ((300, 0), (100, 60)), 128),
    # the same paper's fair share: decodes get up to 30% of the budget, the prompts the rest
    ("fair_share", dict(policy=2, decode_share_pct=30), (500, 70, 1200, 2048, 9, 64), ((400, 0), (90, 0)), 96),
    # the sference post's proposed floor: each admitted prompt gets up to 24 tokens first, the rest
    # is shared, so several prompts are partly prefilled in one step
    ("prefill_floor", dict(prefill_floor=24, max_chunk=80), (300, 700), ((150, 0), (260, 100), (90, 0)), 160),
    # "Chunked Prefill 的 Token 预算" §08/§16: a 25% prefill quota under decode-first, with more
    # decodes than fit beside it, so some decodes wait
    ("quota", dict(prefill_quota_pct=25), tuple(range(100, 3100, 100)), ((500, 0),), 32),
]


@pytest.mark.parametrize("case", POLICY_CASES, ids=[c[0] for c in POLICY_CASES])
def test_policies_every_row_every_step(dev, case):
    """Every row of every step and every written slot against the oracle builder run with the same
    policy; steps with deferred decodes and with several partial prefills."""
    from synth.workloads import _make
    name, cfg, ctx, prompts, budget = case
    w = _make(f"policy_{name}", "bf16", 16, 4, 128, 16, budget, ctx, prompts, 12, 3200 + len(name),
              np.random.default_rng(len(name)))
    gpu = DeviceRun(w, dev, sched_cfg=cfg)
    ora = OracleRun(w, value_device=dev, sched_cfg=cfg)
    seen_partial, seen_deferred = 0, 0
    for step in range(w.steps):
        plan = ora.build()
        meta, out, q_rot = gpu.step()
        torch.cuda.synchronize()
        check_metadata(meta, plan)
        n_prompts = plan["num_seqs"] - plan["num_decodes"]
        seen_partial = max(seen_partial, n_prompts)
        seen_deferred = max(seen_deferred, len(ctx) - plan["num_decodes"])
        say(f"[{w.name}] step {step}: T={plan['num_tokens']} nd={plan['num_decodes']} prompts={n_prompts}")
        if plan["num_tokens"] == 0:
            continue
        check_step_kv_all(gpu, ora, plan, f"step {step}")
        check_outputs(gpu, ora, plan, out, None, f"step {step}")
    if name in ("prefill_floor", "fair_share"):
        assert seen_partial >= 2, "expected several prompts in one step"
    if name in ("prefill_first", "quota"):
        assert seen_deferred > 0, "expected deferred decodes"
