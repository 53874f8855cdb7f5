"""The rotary kernel's arithmetic must not be contracted into fused multiply-adds (each product
and sum is rounded on its own), or K in the cache would not be bit-exact.  Compiles the kernel
for gfx950 to assembly on the host and inspects it.  CPU only (needs hipcc, not a GPU)."""
import os
import re
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "chunked_prefill_mixed_decode_amd", "csrc")


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")), reason="no hipcc")
def test_rope_kernel_has_no_fused_float_multiply_add(tmp_path):
    from chunked_prefill_mixed_decode_amd import build
    out = tmp_path / "rope.s"
    cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{build.INCLUDE}", f"-I{CSRC}", "--cuda-device-only", "-S",
           os.path.join(CSRC, "rope_append.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    asm = out.read_text()
    assert "rope_kv_append_kernel" in asm
    fused = re.findall(r"\b(v_fma_f32|v_fmac_f32\w*|v_mac_f32\w*|v_pk_fma_f32|v_fma_mix\w*)\b", asm)
    assert not fused, f"fused float ops in the rotary kernel: {sorted(set(fused))}"
    assert not re.findall(r"\bv_pk_(mul|add|fma)_f32\b", asm)
