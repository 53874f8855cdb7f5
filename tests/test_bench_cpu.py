"""bench.py's host-side accounting, checked on CPU: the algorithmic bytes and FLOPs its roofline
and chunk figures divide by, against counts written out by hand for a small step, and its refusal
of more than one GPU."""
import os
import subprocess
import sys
import types

import bench
from chunked_prefill_mixed_decode_amd import binding as cb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _two_steps():
    # Two running decodes with 4 and 6 cached tokens (contexts 5 and 7 once their new token is
    # appended) and a 10-token prompt under a budget of 6: each step places both decodes and a
    # 4-token chunk ("Chunked Prefill 的 Token 预算" §03: decodes first, the rest to the prompt).
    s = cb.cb_sched_create(16, 64)
    cb.cb_sched_add_running(s, 4)
    cb.cb_sched_add_running(s, 6)
    cb.cb_sched_add_prompt(s, 10, 0)
    metas = []
    for _ in range(2):
        buf = cb.StepBuffers(8, 16, 64, pin=False)
        metas.append(cb.cb_build_step(s, 6, buf))
    return metas


def test_algorithmic_bytes_and_flops_by_hand():
    w = types.SimpleNamespace(Hq=4, Hkv=2, D=64)
    m0, m1 = _two_steps()
    assert (m0.num_decodes, m0.num_tokens) == (2, 6) and (m1.num_decodes, m1.num_tokens) == (2, 6)
    elt = 2
    kv_row = 2 * 64 * 2 * elt               # K and V of one key: Hkv heads x D x 2 tensors x elt
    qo_row = 2 * 4 * 64 * elt               # q and out of one row: Hq heads x D, read and written
    # step 0: decode keys 5 + 7, chunk rows at positions 0..3 over keys 0..3
    assert bench.decode_bytes(m0, w, elt) == (5 + 7) * kv_row + 2 * qo_row
    assert bench.chunk_bytes(m0, w, elt) == 4 * kv_row + 4 * qo_row
    assert bench.chunk_flops(m0, w) == (1 + 2 + 3 + 4) * 4 * 64 * 4
    # step 1: each decode one key longer; chunk rows at positions 4..7 over keys 0..7
    assert bench.decode_bytes(m1, w, elt) == (6 + 8) * kv_row + 2 * qo_row
    assert bench.chunk_bytes(m1, w, elt) == 8 * kv_row + 4 * qo_row
    assert bench.chunk_flops(m1, w) == (5 + 6 + 7 + 8) * 4 * 64 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout
