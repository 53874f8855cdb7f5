"""The key-coverage inputs of tests/test_gpu_coverage.py can see one lost or doubled stage.

CPU only: the mistake is planted in the oracle's inputs (a 32-key stage's values dropped or
counted twice), and the planted result must fail the bfloat16 bar against the true one, while the
true result rounded to bfloat16 (what a correct kernel returns at best) passes.  Rows at the
longest contexts the GPU test checks: the last chunk row of the long-context layer (264,192 keys)
and a 32,768-key decode.
"""
import numpy as np
import pytest

from oracle import attention as oattn
from oracle.rope import bf16_round
from tests.harness import compare
from tests.test_gpu_coverage import marker_values

Hq, Hkv, D = 64, 8, 128


def attend_marked(P, drop=None, double=None):
    """Zero queries at position P - 1 over marker values of keys 0..P-1; ``drop``/``double`` name
    a stage whose values are removed or counted twice (twice: appended again as extra keys)."""
    v = marker_values(np.arange(P), Hkv, D)
    if drop is not None:
        v[32 * drop:32 * drop + 32] = 0.0
    if double is not None:
        v = np.concatenate([v, v[32 * double:32 * double + 32]])
    n = v.shape[0]
    return oattn.attend(np.zeros((1, Hq, D)), np.zeros((n, Hkv, D), np.float32), v, [n - 1], D ** -0.5)[0]


@pytest.mark.parametrize("P", [264192, 32768])
def test_one_stage_changes_the_result_past_the_bar(P):
    true = attend_marked(P)
    assert compare(bf16_round(true.astype(np.float32)), true, "bf16")[0]
    last = (P - 1) // 32
    for s in (0, last // 2, last):
        assert not compare(attend_marked(P, drop=s), true, "bf16")[0], f"drop stage {s}"
    for s in (last // 3,):
        assert not compare(attend_marked(P, double=s), true, "bf16")[0], f"double stage {s}"
