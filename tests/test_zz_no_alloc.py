"""The attention entry point that allocates nothing (cb_mixed_paged_attention_noalloc, whose
workspace is the library's per-GPU scratch array) against the one that takes a workspace: two
calls in a row, the second on a smaller step, each bit-identical to the workspace call on the same
inputs and within the parity bar of the oracle."""
import numpy as np
import pytest
import torch

from synth import workloads
from tests.harness import DeviceRun, OracleRun, compare, plan_of_meta

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    from chunked_prefill_mixed_decode_amd import binding
    binding._lib()
    return torch.device("cuda:0")


def one_call(dev, w):
    from chunked_prefill_mixed_decode_amd import binding as cb
    g, ora = DeviceRun(w, dev), OracleRun(w, value_device=dev)
    plan = ora.build()
    meta = g.runner.build(g.sched, w.budget)
    assert plan_of_meta(meta)["slot_mapping"] == plan["slot_mapping"]
    dm = g.runner.upload(meta)
    q, k, v = g.step_inputs(meta)
    q_rot = torch.empty_like(q)
    g.runner.append(dm, q, k, v, q_rot)
    kw = dict(num_seqs=meta.num_seqs, num_decodes=meta.num_decodes, max_q_len=meta.max_q_len,
              max_decode_ctx=meta.max_decode_context_len, max_ctx=meta.max_context_len, scale=g.runner.scale)
    args = (q_rot, g.runner.k_cache, g.runner.v_cache, dm["cu_seqlens_q"], dm["context_lens"], dm["cu_blocks"],
            dm["block_table"])
    ws = torch.empty(cb.cb_attn_workspace_bytes(meta.num_seqs, meta.num_decodes, meta.num_tokens, meta.max_q_len,
                                                meta.max_decode_context_len, meta.max_context_len, w.Hq, w.Hkv, w.D),
                     dtype=torch.uint8, device=dev)
    out_ws, out_na = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
    cb.cb_mixed_paged_attention(*args, out_ws, ws, **kw)
    cb.cb_mixed_paged_attention_noalloc(*args, out_na, **kw)
    torch.cuda.synchronize()
    ity = torch.int16 if q.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out_na.view(ity), out_ws.view(ity))
    want = ora.expected_rows(plan)
    rows = sorted(want)
    ok, mabs, _ = compare(out_na.float().cpu().numpy()[rows], np.stack([want[r] for r in rows]), w.dtype)
    print(f"{w.name}: {meta.num_tokens} rows, max|err| {mabs:.3e}", flush=True)
    assert ok
    return meta.num_tokens, ws.numel()


def test_noalloc_matches_workspace_call_twice(dev):
    # the long-context GQA-8 step (decode rows split over many waves), then a smaller MHA step
    t1, b1 = one_call(dev, workloads.small(5))
    t2, b2 = one_call(dev, workloads.small(2))
    assert t2 < t1 and b2 < b1


def test_noalloc_rejects_what_does_not_fit(dev):
    from chunked_prefill_mixed_decode_amd import binding as cb
    lib = cb._lib()
    # a shape whose workspace exceeds the scratch array (many decode rows, 128 heads of one KV head)
    st = torch.cuda.current_stream(dev).cuda_stream
    need = cb.cb_attn_workspace_bytes(60000, 60000, 60000, 1, 64, 64, 128, 1, 128)
    assert need > (64 << 20)
    rc = lib.cb_mixed_paged_attention_noalloc(st, cb.CB_BF16, 60000, 60000, 60000, 1, 64, 64, 128, 1, 128, 16,
                                              0.1, 16, 16, 16, 16, 16, 16, 16, 16)
    assert rc == cb.CB_ERR_CAPACITY
