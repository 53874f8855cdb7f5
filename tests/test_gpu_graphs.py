"""HIP-graph replay of whole steps (runner.StepGraphs) against the eager path, on the GPU.

Each step of a scaled-down workload's cycle runs eagerly, is then captured, and is replayed on
later cycles (from the same builder snapshot, so every step recurs with identical launch
parameters); every replay's attention output and rotated queries must equal the eager run's bit
for bit, with eager torch work and host synchronisations between the replays, and the cache must
hold the same bits afterwards.
"""
import pytest
import torch

from synth import workloads
from tests.gpu_harness import DeviceRun

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return torch.device("cuda:0")


@pytest.mark.parametrize("i", [2, 4])
def test_graph_replay_equals_eager(dev, i):
    from chunked_prefill_mixed_decode_amd.runner import StepGraphs
    w = workloads.small(i)
    g = DeviceRun(w, dev)
    cb = g.cb
    snap = cb.cb_sched_clone(g.sched)
    # Cycle length: steps until the prompts are done, bounded.
    probe, n = cb.cb_sched_clone(snap), 0
    buf = cb.StepBuffers(*g.runner.bufs[0].cap)
    while (w.steps is None and cb.cb_sched_pending_prompts(probe) > 0 or w.steps is not None and n < w.steps) and n < 40:
        cb.cb_build_step(probe, w.budget, buf)
        n += 1
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
    graphs = StepGraphs(g.runner)
    got_q = [torch.empty_like(q) for q in qrots]
    got_o = [torch.empty_like(o) for o in outs]
    modes = []
    for cycle in range(3):
        g.sched = cb.cb_sched_clone(snap)
        for k in range(n):
            meta = g.runner.build(g.sched, w.budget)
            q, kk, vv = inputs[k]

            def launch(dm, k=k, meta=meta, q=q, kk=kk, vv=vv):
                g.runner.append(dm, q, kk, vv, got_q[k])
                g.runner.attend(meta, dm, got_q[k], got_o[k])
            got_o[k].fill_(float("nan"))
            modes.append(graphs.step(meta, launch))
            torch.cuda.synchronize()
            _ = (got_o[k].float() * 2).sum().item()            # eager work between replays
            assert torch.equal(got_o[k].view(torch.int16), outs[k].view(torch.int16)), (cycle, k)
            assert torch.equal(got_q[k].view(torch.int16), qrots[k].view(torch.int16)), (cycle, k)
    assert "replay" in modes and modes.count("captured") == len(graphs.graphs)
    assert torch.equal(g.runner.k_cache.view(torch.int16), kc.view(torch.int16))
    assert torch.equal(g.runner.v_cache.view(torch.int16), vc.view(torch.int16))
