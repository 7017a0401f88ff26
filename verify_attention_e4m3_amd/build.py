"""Build libattn.so (the HIP library behind include/attn.h) in-tree for gfx950.

    python -m verify_attention_e4m3_amd.build

Every build compiles from source; the result is ``verify_attention_e4m3_amd/libattn.so``.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = [os.path.join(CSRC, "attn_kernels.hip"), os.path.join(CSRC, "prefill_kernels.hip"),
           os.path.join(CSRC, "attn_plan.cpp")]
# Measurement-only library used by bench.py (a plain streaming-read kernel); not the attention ABI.
PROBE_LIB = os.path.join(PKG, "libattn_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "stream_probe.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def command(out: str = LIB, sources=None) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
        # packed FP32 VALU ops stay off in all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-inline-asm", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *(sources or SOURCES), "-o", out,
    ]


def _compile(out: str, sources, verbose: bool):
    tmp = out + ".tmp"
    cmd = command(tmp, sources)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(LIB, SOURCES, verbose)
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
