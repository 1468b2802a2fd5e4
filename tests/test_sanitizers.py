"""Host sanitizer runs (no GPU): the CPU oracle and libnf4's C-ABI validation
layer built with AddressSanitizer and UndefinedBehaviorSanitizer (on host code
only: every -fsanitize follows -Xarch_host; device code is built as usual) and
driven over their entry points with edge-case and out-of-range arguments.  Any
sanitizer report fails the run (-fno-sanitize-recover)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "dequant_gemv_nf4_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "oracle_asan")
    rc, out = _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(HERE, "oracle_driver.cpp"),
                    os.path.join(ROOT, "oracle", "nf4_oracle.cpp"), "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=600)
    assert rc == 0 and "oracle sanitizer run: ok" in out, out


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("no hipcc")
    exe = str(tmp_path / "abi_asan")
    srcs = [os.path.join(CSRC, f) for f in ("api.hip", "ring.hip", "pack.hip", "gemv.hip",
                                            "gemm_mfma.hip", "gemm_prefill.hip", "embed.hip")]
    srcs.append(os.path.join(HERE, "abi_driver.cpp"))
    flags = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include")]
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]

    def compile_one(so):
        s, o = so
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        return _run([HIPCC] + flags + ["-c"] + lang + [s, "-o", o], timeout=600)
    with ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 1)) as ex:
        for rc, out in ex.map(compile_one, zip(srcs, objs)):
            assert rc == 0, out
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined"] + objs + ["-o", exe], timeout=600)
    assert rc == 0, out
    env = dict(ENV, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    rc, out = _run([exe], env=env, timeout=600)
    assert rc == 0 and "abi sanitizer run: ok" in out, out
