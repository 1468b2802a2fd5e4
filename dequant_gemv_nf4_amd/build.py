"""Build libnf4.so (HIP, gfx950) in-tree with hipcc.

One shared library holds every kernel and the C ABI of include/nf4.h.  Each
source is compiled to an object in parallel, then the objects are linked.
Packed FP32 instructions are switched off for all device code.  Kernel
arguments are preloaded into scalar registers (up to 16 words, gfx950 supports
it), so a wave does not wait on an argument load before its first memory
requests.
"""
import hashlib
import json
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnf4.so")
SOURCES = ["api.hip", "pack.hip", "gemv.hip", "gemm_mfma.hip", "gemm_prefill.hip", "embed.hip",
           "ring.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# what the library is built from (the hash the benchmark line reports)
HASHED = ["include/nf4.h"] + ["dequant_gemv_nf4_amd/csrc/" + f for f in
                              ("api.hip", "nf4_device.h", "nf4_launch.h", "nf4_split.h",
                               "pack.hip", "gemv.hip", "gemm_mfma.hip", "gemm_prefill.hip",
                               "embed.hip", "ring.hip")]
BUILD_INFO = os.path.join(HERE, "build_info.json")


def sources_sha256() -> str:
    h = hashlib.sha256()
    for f in HASHED:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _git(*args):
    try:
        r = subprocess.run(["git", "-C", ROOT] + list(args), capture_output=True, text=True,
                           timeout=10)
        return r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def write_build_info():
    """Record what the library was built from (commit, sources, toolchain) beside it."""
    info = {"git_head": _git("rev-parse", "HEAD"),
            "git_dirty": bool(_git("status", "--porcelain", "--untracked-files=no")),
            "sources_sha256": sources_sha256(),
            "hipcc": (subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
                      .stdout.splitlines() or [None])[0]}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)
    return info
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-kernarg-preload-count=16",
         "-I", os.path.join(ROOT, "include"), "-Wall"]


def compile_command(src: str, obj: str):
    return [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs, out: str):
    return [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", out] + list(objs)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="nf4build_") as tmpdir:
        objs = [os.path.join(tmpdir, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [compile_command(s, o) for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = min(len(cmds), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True),
                                  cmds))
        for c, r in zip(cmds, results):
            out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                            if "packed-fp32-ops" not in l)
            if out.strip():
                print(out, file=sys.stderr, flush=True)
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, c)
        tmp = LIB + ".tmp"
        link = link_command(objs, tmp)
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    write_build_info()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
