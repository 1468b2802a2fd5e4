"""Streaming-read probe for the benchmark: the floor a product launch over
packed weights is compared with (a plain kernel that reads the same codes and
scales bytes once and writes the same output bytes; probe/stream_probe.hip).

Measurement aid only: bench.py uses it; the product library does not.
"""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "libnf4probe.so")
SRC = os.path.join(_HERE, "stream_probe.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
_lib = None


def build_command(out):
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
            "-I", _HERE, "-o", out, SRC]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{msg}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        L.nf4_probe_variants.restype = ctypes.c_int
        L.nf4_probe_stream.restype = ctypes.c_int
        L.nf4_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_void_p]
        _lib = L
    return _lib


def variants():
    return int(lib().nf4_probe_variants())


def stream(codes, scales, out, variant, stream_handle):
    """Enqueue one probe launch over the bytes of `codes` and `scales` (device
    tensors) writing `out` (device tensor of 32-bit words)."""
    r = lib().nf4_probe_stream(ctypes.c_void_p(codes.data_ptr()), codes.numel() * codes.element_size(),
                               ctypes.c_void_p(scales.data_ptr()),
                               scales.numel() * scales.element_size(),
                               ctypes.c_void_p(out.data_ptr()), out.numel(), int(variant),
                               ctypes.c_void_p(stream_handle))
    if r != 0:
        raise RuntimeError(f"nf4_probe_stream returned {r}")
