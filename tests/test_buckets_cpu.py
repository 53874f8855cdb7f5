"""Padded launch shapes (runner.Buckets) on the host: what build() writes and plans, no GPU."""
import pytest
import torch

from chunked_prefill_mixed_decode_amd import binding as cb
from chunked_prefill_mixed_decode_amd.runner import Buckets, MixedStepRunner, round_up


def _runner(cap_tokens=512):
    return MixedStepRunner(Hq=8, Hkv=2, D=64, block_size=16, num_blocks=256, dtype=torch.float32,
                           device="cpu", max_pos=8192, cap_seqs=16, cap_tokens=cap_tokens,
                           cap_blocks=512, sentinel=False)


def _sched():
    s = cb.cb_sched_create(16, 256)
    for c in (700, 33, 1500):
        cb.cb_sched_add_running(s, c)
    cb.cb_sched_add_prompt(s, 900, 0)
    return s


def test_round_up():
    assert [round_up(x, 64) for x in (0, 1, 64, 65, 130)] == [0, 64, 64, 128, 192]
    assert round_up(37, 0) == 37


def test_bucketed_build_pads_rows_and_bounds():
    r = _runner()
    exact = r.build(_sched(), 100)
    padded = r.build(_sched(), 100, buckets=Buckets(tokens=64, context=1024))
    T = exact.num_tokens
    assert T == 100 and padded.num_tokens == T and exact.launch_tokens == T
    assert padded.launch_tokens == 128
    # the builder's own output is unchanged; rows [T, 128) carry position and slot -1
    buf = r.bufs[padded.buf_index].arrays
    assert torch.equal(buf["positions"][:T], exact.host["positions"])
    assert (buf["positions"][T:128] == -1).all() and (buf["slot_mapping"][T:128] == -1).all()
    assert padded.exact_max == (exact.max_q_len, exact.max_context_len, exact.max_decode_context_len)
    assert padded.max_q_len == min(round_up(exact.max_q_len, 64), 128)
    assert padded.max_context_len == round_up(exact.max_context_len, 1024)
    assert padded.max_decode_context_len == round_up(exact.max_decode_context_len, 1024)
    # the decode split is planned for the padded launch shape
    S, nd = padded.num_seqs, padded.num_decodes
    want = torch.full((cb.cb_decode_plan_ints(nd, padded.plan_waves),), -7, dtype=torch.int32)
    cb.cb_decode_plan(padded.host["cu_seqlens_q"], padded.host["context_lens"], nd, padded.max_q_len,
                      padded.max_context_len, 8, 2, want, None)
    got = r.bufs[padded.buf_index].arrays["decode_plan"][:want.numel()]
    head = 4 + nd + 1
    W = int(want[2])
    assert torch.equal(got[:head + W], want[:head + W])
    assert torch.equal(got[head + padded.plan_waves:head + padded.plan_waves + W + 1],
                       want[head + padded.plan_waves:head + padded.plan_waves + W + 1])
    # the workspace is sized for the padded rows
    assert r.workspace_bytes(padded) >= r.workspace_bytes(exact)


def test_bucket_never_exceeds_capacity():
    r = _runner(cap_tokens=100)
    m = r.build(_sched(), 100, buckets=Buckets(tokens=64, context=1024))
    assert m.num_tokens == 100 and m.launch_tokens == 100


def test_runner_refuses_a_step_beyond_the_rotary_table():
    # The rotary/append kernel skips rows whose position lies past its table (the padding rows'
    # convention), so a serving loop that outgrows max_pos must be stopped on the host.
    import types
    from chunked_prefill_mixed_decode_amd import runner as rn
    r = types.SimpleNamespace(ring=0, copied=[None, None], bufs=[cb.StepBuffers(4, 16, 16, pin=False)] * 2,
                              cos_sin=torch.zeros((19, 64)), Hq=2, Hkv=2, device=torch.device("cpu"))
    s = cb.cb_sched_create(16, 8)
    cb.cb_sched_add_running(s, 19)          # its query sits at position 19, past a 19-row table
    with pytest.raises(ValueError, match="rotary table"):
        rn.MixedStepRunner.build(r, s, 8)
