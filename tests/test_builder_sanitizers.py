"""The host batch builder (csrc/sched.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/native/builder_fuzz.cpp drives it through the C ABI over random configurations, set-ups,
budgets and capacities (every error path), finishes and clones, and checks the invariants a caller
relies on.  Host code only (g++); skipped when g++ is not installed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_builder_fuzz_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not installed")
    exe = str(tmp_path / "builder_fuzz")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-static-libasan", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "native", "builder_fuzz.cpp"),
                    os.path.join(ROOT, "chunked_prefill_mixed_decode_amd", "csrc", "sched.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "600"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok:"), r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
