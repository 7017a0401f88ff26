"""Build checks without a GPU: every device kernel of the library compiles for gfx950 with no
scratch (no register spills), read from the compiler's resource-usage remarks."""
import os
import re
import subprocess

import pytest

from verify_attention_e4m3_amd import build as B


@pytest.mark.parametrize("source", ["attn_kernels.hip", "prefill_kernels.hip"])
def test_kernels_use_no_scratch(source, tmp_path):
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "--offload-device-only", "-c",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-inline-asm",
           "-Wno-unused-command-line-argument", "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC, os.path.join(B.CSRC, source),
           "-o", str(tmp_path / "k.o")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = re.findall(r"Function Name: (\S+)", res.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", res.stderr)]
    assert kernels and len(scratch) == len(kernels), res.stderr[-2000:]
    spilling = [k for k, s in zip(kernels, scratch) if s != 0]
    assert not spilling, spilling
