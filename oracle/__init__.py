"""Python view of the plain fp64 CPU oracle (oracle/nf4_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package's smoke() check and
by bench.py's cpu_baseline leg.  The product library never imports it, and it
never imports the product.  All arrays are numpy, on the host.

Parity status of each function (what pins it, see tests/test_oracle.py):
  normal_quantile   pinned: statistics.NormalDist / scipy ndtri library routines
  codebook          pinned: invariants + QLoRA paper's printed NF4 table (1e-6)
  f32_to_f16_bits   pinned: numpy float16 conversion, hand values
  quantize          pinned: brute-force nearest level on 2x64 and adversarial
                    values, round trip, error bound, scale invariance, zero group
  pack/unpack       pinned: hand byte vector, size ratio of the README
  dequant_f64/f32   pinned: exact special codes, numpy fp32 multiply
  gemm_rows         pinned: numpy fp64 matmul on tiny inputs, closed forms
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

STATUS_NONFINITE = 1
STATUS_SCALE_OVERFLOW = 2

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def lib():
    """Load liboracle.so, building it with g++ if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_normal_quantile.restype = ctypes.c_double
        L.orc_normal_quantile.argtypes = [ctypes.c_double]
        L.orc_codebook.restype = None
        L.orc_codebook.argtypes = [_f64p, _f32p]
        L.orc_f32_to_f16_bits.restype = ctypes.c_uint16
        L.orc_f32_to_f16_bits.argtypes = [ctypes.c_float]
        L.orc_f16_bits_to_f64.restype = ctypes.c_double
        L.orc_f16_bits_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_bits_to_f64.restype = ctypes.c_double
        L.orc_bf16_bits_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_quantize.restype = ctypes.c_int32
        L.orc_quantize.argtypes = [_f32p, _i64, _i64, _u8p, _u16p]
        L.orc_pack.restype = None
        L.orc_pack.argtypes = [_u8p, _i64, _i64, _u8p]
        L.orc_unpack_codes.restype = None
        L.orc_unpack_codes.argtypes = [_u8p, _i64, _i64, _u8p]
        L.orc_dequant_f64.restype = None
        L.orc_dequant_f64.argtypes = [_u8p, _u16p, _i64, _i64, _f64p]
        L.orc_dequant_f32.restype = None
        L.orc_dequant_f32.argtypes = [_u8p, _u16p, _i64, _i64, _f32p]
        L.orc_gemm_rows.restype = None
        L.orc_gemm_rows.argtypes = [_u8p, _u16p, _i64, _i64, _u16p, _i64, _i64p,
                                    _i64, _f64p, _f64p]
        L.orc_f64_to_bf16_bits.restype = ctypes.c_uint16
        L.orc_f64_to_bf16_bits.argtypes = [ctypes.c_double]
        L.orc_embed.restype = ctypes.c_int32
        L.orc_embed.argtypes = [_u8p, _u16p, _i64, _i64, _i64p, _i64, _u16p]
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def normal_quantile(p: float) -> float:
    return lib().orc_normal_quantile(float(p))


def codebook():
    """(levels fp64 [16], levels fp32 [16])."""
    l64 = np.zeros(16, np.float64)
    l32 = np.zeros(16, np.float32)
    lib().orc_codebook(_p(l64, _f64p), _p(l32, _f32p))
    return l64, l32


def f32_to_f16_bits(f: float) -> int:
    return int(lib().orc_f32_to_f16_bits(ctypes.c_float(float(np.float32(f)))))


def f16_bits_to_f64(h: int) -> float:
    return lib().orc_f16_bits_to_f64(int(h))


def bf16_bits_to_f64(b: int) -> float:
    return lib().orc_bf16_bits_to_f64(int(b))


def quantize(W):
    """W fp32 [N][K] -> (codes uint8 [N][K] one per byte, scales uint16 [N][K/64], status)."""
    W = _c(W, np.float32)
    N, K = W.shape
    assert K % 64 == 0
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, K // 64), np.uint16)
    st = lib().orc_quantize(_p(W, _f32p), N, K, _p(codes, _u8p), _p(scales, _u16p))
    return codes, scales, int(st)


def pack(codes):
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    out = np.zeros((N, K // 2), np.uint8)
    lib().orc_pack(_p(codes, _u8p), N, K, _p(out, _u8p))
    return out


def unpack_codes(packed):
    packed = _c(packed, np.uint8)
    N, K2 = packed.shape
    out = np.zeros((N, 2 * K2), np.uint8)
    lib().orc_unpack_codes(_p(packed, _u8p), N, 2 * K2, _p(out, _u8p))
    return out


def quantize_pack(W):
    """W -> (packed codes [N][K/2], scales [N][K/64], status)."""
    codes, scales, st = quantize(W)
    return pack(codes), scales, st


def dequant_f64(packed, scales):
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    N, K2 = packed.shape
    out = np.zeros((N, 2 * K2), np.float64)
    lib().orc_dequant_f64(_p(packed, _u8p), _p(scales, _u16p), N, 2 * K2, _p(out, _f64p))
    return out


def dequant_f32(packed, scales):
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    N, K2 = packed.shape
    out = np.zeros((N, 2 * K2), np.float32)
    lib().orc_dequant_f32(_p(packed, _u8p), _p(scales, _u16p), N, 2 * K2, _p(out, _f32p))
    return out


def gemm(packed, scales, X, rows=None):
    """X bf16 bits uint16 [M][K] (or [K]) -> (Y fp64 [M][R], A = sum|w x| [M][R]).

    R = len(rows) if rows is given, else N.
    """
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    X = _c(X, np.uint16)
    if X.ndim == 1:
        X = X[None, :]
    N, K2 = packed.shape
    K = 2 * K2
    M = X.shape[0]
    assert X.shape[1] == K
    if rows is None:
        rp = None
        R = N
    else:
        rows = _c(rows, np.int64)
        assert rows.min() >= 0 and rows.max() < N
        rp = _p(rows, _i64p)
        R = len(rows)
    Y = np.zeros((M, R), np.float64)
    A = np.zeros((M, R), np.float64)
    lib().orc_gemm_rows(_p(packed, _u8p), _p(scales, _u16p), N, K, _p(X, _u16p), M, rp, R,
                        _p(Y, _f64p), _p(A, _f64p))
    return Y, A


# tolerance stated for the fp32 GPU outputs: per element
#   |y - y_ref| <= REL_TOL * sum_k |w~_k x_k| + ABS_TOL
REL_TOL = 2e-3
ABS_TOL = 1e-5


def within_tolerance(y, y_ref, absum):
    """Boolean mask of elements meeting the per-element tolerance (fp64 bound)."""
    y = np.asarray(y, np.float64)
    return np.abs(y - y_ref) <= REL_TOL * absum + ABS_TOL


def f64_to_bf16_bits(v: float) -> int:
    """Nearest bfloat16 to v (ties to even), as bits; NaN -> 0x7FC0."""
    return int(lib().orc_f64_to_bf16_bits(float(v)))


EMBED_BAD_ID = 1


def embed(packed, scales, ids):
    """Rows ids of the dequantised matrix rounded once to bf16 -> (uint16 bits
    [T][K], status).  Out-of-range ids give zero rows and status EMBED_BAD_ID."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    ids = _c(ids, np.int64).reshape(-1)
    N, K = packed.shape[0], packed.shape[1] * 2
    out = np.empty((ids.size, K), np.uint16)
    st = lib().orc_embed(_p(packed, _u8p), _p(scales, _u16p), N, K, _p(ids, _i64p),
                         ids.size, _p(out, _u16p))
    return out, int(st)
