"""GPU parity on seeded random small workloads: every row of every step against the oracle.

Each case draws a head geometry (group width 1 to 16, 1 to 3 KV heads, head dim 64 or 128), a
block size (8 to 256), the element type (bf16, or float32 one time in five), 0 to 6 running
decodes with contexts U[1, 1500], 1 to 3 prompts of U[1, 900] tokens (some with a cached prefix)
and a token budget that leaves room for a chunk beside the decodes, then runs the workload until
every prompt has had its last chunk.  Every step: metadata and every written K/V slot bit-exact,
the rotated queries bit-exact, every output row within the tolerance of its element type; then
the step's chunk rows launched alone (their own key split and combine), every row again.  Beside
them, random shapes through cb_linear against its rigorous bound.
"""
import numpy as np
import pytest
import torch

from synth import workloads
from tests.harness import DeviceRun, OracleRun
from tests.test_gpu_chunk_only import chunk_only
from tests.test_gpu_parity import check_metadata, check_outputs, check_q_rot, check_step_kv, say

pytestmark = pytest.mark.gpu

CASES = 48


def fuzz_workload(seed: int) -> workloads.Workload:
    rng = np.random.Generator(np.random.PCG64(5000 + seed))
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 7, 8, 16]))
    Hkv = int(rng.integers(1, 3, endpoint=True))
    bs = int(rng.choice([8, 16, 32, 64, 256]))
    nd = int(rng.integers(0, 6, endpoint=True))
    ctx = rng.integers(1, 1500, size=nd, endpoint=True)
    n_prompts = int(rng.integers(1, 3, endpoint=True))
    prompts = []
    for _ in range(n_prompts):
        L = int(rng.integers(1, 900, endpoint=True))
        cached = int(rng.integers(0, L - 1, endpoint=True)) if (L > 1 and rng.random() < 0.4) else 0
        prompts.append((L, cached))
    todo = sum(L - c for L, c in prompts)
    budget = nd + max(1, int(rng.integers(max(16, todo // 8), max(17, todo // 2), endpoint=True)))
    return workloads._make(f"fuzz{seed}_{dtype}_g{G}x{Hkv}_d{D}_bs{bs}", dtype, G * Hkv, Hkv, D, bs, budget, ctx,
                           prompts, None, 5000 + seed, rng, max_steps=32)


def run_step(g: DeviceRun):
    """One step (build, pull, rope + append, attention); returns the metadata, its device views,
    the output and the rotated queries."""
    g.arrive(g.step_index)
    g.step_index += 1
    meta = g.runner.build(g.sched, g.w.budget)
    dm = g.runner.upload(meta)
    q, k, v = g.step_inputs(meta)
    q_rot, out = torch.empty_like(q), torch.empty_like(q)
    g.runner.append(dm, q, k, v, q_rot)
    g.runner.attend(meta, dm, q_rot, out)
    g.written += meta.num_tokens
    return meta, dm, out, q_rot


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    from chunked_prefill_mixed_decode_amd import binding
    binding._lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("seed", range(CASES))
def test_fuzz_workload_every_row_every_step(dev, seed):
    w = fuzz_workload(seed)
    say(f"[{w.name}] decodes {list(w.decode_ctx)}, prompts {list(w.prompts)}, budget {w.budget}")
    gpu = DeviceRun(w, dev)
    ora = OracleRun(w, value_device=dev)
    step = 0
    while ora.b.pending_prompts() > 0:
        plan = ora.build()
        meta, dm, out, q_rot = run_step(gpu)
        torch.cuda.synchronize()
        check_metadata(meta, plan)
        rows = set(range(plan["num_tokens"]))
        check_step_kv(gpu, ora, plan, rows)
        check_q_rot(gpu, ora, plan, q_rot, rows)
        check_outputs(gpu, ora, plan, out, None, f"step {step}")
        nd, T = plan["num_decodes"], plan["num_tokens"]
        if T > nd and nd > 0:                 # (without decodes the step itself was chunk-only)
            alone = torch.zeros_like(out)
            alone[nd:] = chunk_only(gpu, meta, dm, q_rot)
            check_outputs(gpu, ora, plan, alone, set(range(nd, T)), f"step {step}, chunk rows alone")
        step += 1
        assert step <= w.max_steps


POLICY_CASES = 16


def fuzz_policy(seed: int) -> dict:
    """A random builder configuration: the priority order (decode-first, prefill-first, fair share
    with a random decode share), and sometimes a per-request chunk cap, a prefill floor, a cap on
    partial prefills per step and a prefill quota."""
    rng = np.random.Generator(np.random.PCG64(6000 + seed))
    cfg = {"policy": int(rng.integers(0, 2, endpoint=True))}
    if cfg["policy"] == 2:
        cfg["decode_share_pct"] = int(rng.integers(10, 60, endpoint=True))
    if rng.random() < 0.5:
        cfg["max_chunk"] = int(rng.integers(16, 200, endpoint=True))
    if rng.random() < 0.5:
        cfg["prefill_floor"] = int(rng.integers(8, 64, endpoint=True))
    if rng.random() < 0.3:
        cfg["max_partial_prefills"] = int(rng.integers(1, 3, endpoint=True))
    if cfg["policy"] == 0 and rng.random() < 0.4:
        cfg["prefill_quota_pct"] = int(rng.integers(10, 50, endpoint=True))
    return cfg


@pytest.mark.parametrize("seed", range(POLICY_CASES))
def test_fuzz_policies_every_row_every_step(dev, seed):
    """The random workloads under random builder configurations (deferred decodes, several partial
    prefills per step, capped chunks): every row of every step against the oracle builder run
    with the same configuration."""
    w = fuzz_workload(100 + seed)
    cfg = fuzz_policy(seed)
    say(f"[{w.name}] {cfg}, decodes {list(w.decode_ctx)}, prompts {list(w.prompts)}, budget {w.budget}")
    gpu = DeviceRun(w, dev, sched_cfg=cfg)
    ora = OracleRun(w, value_device=dev, sched_cfg=cfg)
    step = 0
    while ora.b.pending_prompts() > 0:
        plan = ora.build()
        meta, dm, out, q_rot = run_step(gpu)
        torch.cuda.synchronize()
        check_metadata(meta, plan)
        if plan["num_tokens"]:
            rows = set(range(plan["num_tokens"]))
            check_step_kv(gpu, ora, plan, rows)
            check_q_rot(gpu, ora, plan, q_rot, rows)
            check_outputs(gpu, ora, plan, out, None, f"step {step}")
        step += 1
        assert step <= w.max_steps


LINEAR_CASES = 8


@pytest.mark.parametrize("seed", range(LINEAR_CASES))
def test_fuzz_linear_shapes(dev, seed):
    from chunked_prefill_mixed_decode_amd import binding as cb
    from tests.test_gpu_linear import _check, _inputs, _ws
    rng = np.random.default_rng(7000 + seed)
    while True:
        M = int(rng.integers(1, 1100, endpoint=True))
        N = 128 * int(rng.integers(1, 96, endpoint=True))
        K = 64 * int(rng.integers(1, 64, endpoint=True))
        if M * N * K <= 2_000_000_000:
            break
    x, w = _inputs(M, N, K, dev, seed=20 + seed)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    cb.cb_linear(x, w, y, _ws(M, N, K, dev))
    torch.cuda.synchronize()
    _check(x, w, y)
