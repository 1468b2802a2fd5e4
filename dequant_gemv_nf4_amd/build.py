"""Build libnf4.so (HIP, gfx950) in-tree with hipcc.

One shared library holds every kernel and the C ABI of include/nf4.h.  Packed
FP32 instructions are switched off for all device code.  Kernel arguments are
preloaded into scalar registers (up to 14 words, gfx950 supports it), so a wave
does not wait on an argument load before its first memory requests.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnf4.so")
SOURCES = ["api.hip", "pack.hip", "gemv.hip", "gemm_mfma.hip", "gemm_prefill.hip", "embed.hip", "ring.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def command(out: str):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-I", os.path.join(ROOT, "include"), "-Wall",
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
