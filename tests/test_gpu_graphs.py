"""HIP-graph replay of whole steps (runner.StepGraphs) on the GPU, against the oracle and the
eager path.

Each step of a scaled-down workload's cycle runs eagerly, is then captured, and is replayed on
later cycles (from the same builder snapshot, so every step recurs with identical launch
parameters); every replay's attention output must agree with the oracle's (fp64, non-chunked) at
the parity bar and equal the eager run's bit for bit, its rotated queries likewise, with eager
torch work and host synchronisations between the replays, and the cache must hold the same bits
afterwards.
"""
import numpy as np
import pytest
import torch

from synth import workloads
from tests.gpu_harness import DeviceRun
from tests.harness import OracleRun, compare


def oracle_cycle(w, dev, n):
    """The oracle's outputs for every row of the cycle's first n steps: [T, Hq, D] per step."""
    ora = OracleRun(w, value_device=dev)
    outs = []
    for _ in range(n):
        plan = ora.build()
        want = ora.expected_rows(plan)
        outs.append(np.stack([want[r] for r in range(plan["num_tokens"])]))
    return outs


def check_oracle(got, want, dtype, tag):
    ok, mabs, mrel = compare(got.float().cpu().numpy(), want, dtype)
    assert ok, f"{tag}: max abs {mabs}, max rel {mrel}"

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return torch.device("cuda:0")


def _cycle_len(g, snap) -> int:
    """Steps until the prompts are done (or the workload's step count), at most 40."""
    w, cb = g.w, g.cb
    probe, n = cb.cb_sched_clone(snap), 0
    buf = cb.StepBuffers(*g.runner.bufs[0].cap)
    while (w.steps is None and cb.cb_sched_pending_prompts(probe) > 0 or w.steps is not None and n < w.steps) and n < 40:
        cb.cb_build_step(probe, w.budget, buf)
        n += 1
    return n


@pytest.mark.parametrize("i", [2, 4, 9])
def test_graph_replay_equals_eager(dev, i):
    from chunked_prefill_mixed_decode_amd.runner import StepGraphs
    w = workloads.small(i)
    g = DeviceRun(w, dev)
    cb = g.cb
    snap = cb.cb_sched_clone(g.sched)
    n = _cycle_len(g, snap)
    # Eager reference: inputs and outputs per step (fixed addresses, reused by the graphs).
    metas, inputs, qrots, outs = [], [], [], []
    g.sched = cb.cb_sched_clone(snap)
    for k in range(n):
        meta, out, q_rot = g.step()
        torch.cuda.synchronize()
        metas.append(meta)
        inputs.append(g.step_inputs(meta))
        qrots.append(q_rot.clone())
        outs.append(out.clone())
    ws = max(g.runner.workspace_bytes(m) for m in metas)
    g.runner.ensure_workspace(ws)
    kc, vc = g.runner.k_cache.clone(), g.runner.v_cache.clone()
    want = oracle_cycle(w, dev, n)
    graphs = StepGraphs(g.runner)
    got_q = [torch.empty_like(q) for q in qrots]
    got_o = [torch.empty_like(o) for o in outs]
    modes = []
    for cycle in range(3):
        g.sched = cb.cb_sched_clone(snap)
        for k in range(n):
            g.arrive(k)
            meta = g.runner.build(g.sched, w.budget)
            q, kk, vv = inputs[k]

            def launch(dm, k=k, meta=meta, q=q, kk=kk, vv=vv):
                g.runner.append(dm, q, kk, vv, got_q[k])
                g.runner.attend(meta, dm, got_q[k], got_o[k])
            got_o[k].fill_(float("nan"))
            modes.append(graphs.step(meta, launch))
            torch.cuda.synchronize()
            _ = (got_o[k].float() * 2).sum().item()            # eager work between replays
            check_oracle(got_o[k], want[k], w.dtype, f"cycle {cycle} step {k}")
            assert torch.equal(got_o[k].view(torch.int16), outs[k].view(torch.int16)), (cycle, k)
            assert torch.equal(got_q[k].view(torch.int16), qrots[k].view(torch.int16)), (cycle, k)
    assert "replay" in modes and modes.count("captured") == len(graphs.graphs)
    assert torch.equal(g.runner.k_cache.view(torch.int16), kc.view(torch.int16))
    assert torch.equal(g.runner.v_cache.view(torch.int16), vc.view(torch.int16))


@pytest.mark.parametrize("i", [2, 4, 9])
def test_bucketed_graph_replay(dev, i):
    # Padded launch shapes (runner.Buckets): steps that round to the same shape share one graph
    # (and one set of row buffers of the padded length).  Rows [0, T) of every replay equal an
    # eager run of the same padded launch bit for bit, and the unpadded eager step within the
    # output tolerance (a larger context bound may choose other key splits); the padding rows
    # append nothing, so the cache ends bit-identical to the unpadded run's.
    from chunked_prefill_mixed_decode_amd.runner import Buckets, StepGraphs
    w = workloads.small(i)
    g = DeviceRun(w, dev)
    cb = g.cb
    snap = cb.cb_sched_clone(g.sched)
    n = _cycle_len(g, snap)
    ref, inputs, exact = [], [], set()
    for k in range(n):
        meta, out, _ = g.step()
        torch.cuda.synchronize()
        inputs.append(g.step_inputs(meta))
        ref.append(out.clone())
        exact.add(StepGraphs.key(meta)[1:])          # launch shape without the pinned buffer
    kc, vc = g.runner.k_cache.clone(), g.runner.v_cache.clone()
    want = oracle_cycle(w, dev, n)
    b = Buckets(tokens=64, context=256)
    tol = dict(atol=2e-2, rtol=1e-2) if g.dtype == torch.bfloat16 else dict(atol=1e-4, rtol=0)

    def padded_meta(sched):
        meta = g.runner.build(sched, w.budget, buckets=b)
        assert meta.launch_tokens % 64 == 0 or meta.launch_tokens == g.runner.bufs[0].cap[1]
        assert meta.launch_tokens >= meta.num_tokens
        return meta

    # Eager runs of the padded launches (and the workspace they need).
    g.sched = cb.cb_sched_clone(snap)
    padded, metas = [], []
    for k in range(n):
        g.arrive(k)
        meta = padded_meta(g.sched)
        T, Tp = meta.num_tokens, meta.launch_tokens
        q, kk, vv = (torch.cat([x, x.new_zeros((Tp - T,) + x.shape[1:])]) for x in inputs[k])
        q_rot, out = torch.empty_like(q), torch.empty_like(q)
        dm = g.runner.upload(meta)
        g.runner.append(dm, q, kk, vv, q_rot)
        g.runner.attend(meta, dm, q_rot, out)
        torch.cuda.synchronize()
        padded.append(out[:T].clone())
        metas.append(meta)
        torch.testing.assert_close(out[:T].float(), ref[k].float(), **tol)
    g.runner.ensure_workspace(max(g.runner.workspace_bytes(m) for m in metas))
    graphs = StepGraphs(g.runner)
    rows = {}                                       # graph key -> row buffers at fixed addresses
    modes = []
    for cycle in range(3):
        g.sched = cb.cb_sched_clone(snap)
        for k in range(n):
            g.arrive(k)
            meta = padded_meta(g.sched)
            T, Tp = meta.num_tokens, meta.launch_tokens
            key = StepGraphs.key(meta)
            if key not in rows:
                rows[key] = [torch.zeros((Tp,) + x.shape[1:], dtype=x.dtype, device=dev) for x in inputs[k]]
                rows[key] += [torch.empty_like(rows[key][0]), torch.empty_like(rows[key][0])]
            q, kk, vv, q_rot, out = rows[key]
            for dst, src in zip((q, kk, vv), inputs[k]):
                dst[:T].copy_(src)
            out.fill_(float("nan"))

            def launch(dm, meta=meta, q=q, kk=kk, vv=vv, q_rot=q_rot, out=out):
                g.runner.append(dm, q, kk, vv, q_rot)
                g.runner.attend(meta, dm, q_rot, out)
            modes.append(graphs.step(meta, launch))
            torch.cuda.synchronize()
            _ = (out[:T].float() * 2).sum().item()                  # eager work between replays
            check_oracle(out[:T], want[k], w.dtype, f"bucketed cycle {cycle} step {k}")
            assert torch.equal(out[:T].view(torch.int16), padded[k].view(torch.int16)), (cycle, k)
    # One graph per (pinned buffer, padded shape); no more padded shapes than exact ones.
    shapes = {key[1:] for key in graphs.graphs}
    assert "replay" in modes and modes.count("captured") == len(graphs.graphs)
    assert len(shapes) <= len(exact) and len(graphs.graphs) <= 2 * len(shapes)
    assert torch.equal(g.runner.k_cache.view(torch.int16), kc.view(torch.int16))
    assert torch.equal(g.runner.v_cache.view(torch.int16), vc.view(torch.int16))
