"""Host-side checks of libnf4.so that need no GPU: it loads, exports every symbol
include/nf4.h declares, its codebook equals the oracle's bit for bit, and its
argument validation returns the documented status codes before touching a
device."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4.h")
LIB = os.path.join(ROOT, "dequant_gemv_nf4_amd", "libnf4.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf4_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libnf4.so is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.nf4_pack.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    L.nf4_unpack.argtypes = [vp, vp, i64, i64, vp, vp]
    L.nf4_gemv.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.nf4_gemm_smallm.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
    L.nf4_gemm_prefill.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
    L.nf4_gemm_smallm_ws.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, i64, vp]
    L.nf4_gemm_smallm_workspace_bytes.argtypes = [i64, i64, i64]
    L.nf4_gemm_smallm_workspace_bytes.restype = ctypes.c_int64
    L.nf4_gemm_prefill_ws.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, i64, vp]
    L.nf4_gemm_prefill_workspace_bytes.argtypes = [i64, i64, i64]
    L.nf4_gemm_prefill_workspace_bytes.restype = ctypes.c_int64
    L.nf4_embed.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, vp]
    L.nf4_ring_create.argtypes = [ctypes.POINTER(ctypes.c_void_p), vp, vp, i64, vp, vp]
    L.nf4_ring_gemm.argtypes = [vp, vp, vp, i64, i64, vp, i64, vp]
    L.nf4_ring_destroy.argtypes = [vp]
    L.nf4_ring_slot_bytes.argtypes = [i64, i64]
    L.nf4_ring_slot_bytes.restype = ctypes.c_int64
    L.nf4_strerror.restype = ctypes.c_char_p
    return L


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("nf4_pack", "nf4_unpack", "nf4_gemv", "nf4_gemm_smallm", "nf4_gemm_prefill",
                     "nf4_gemm_smallm_ws", "nf4_gemm_smallm_workspace_bytes",
                     "nf4_gemm_prefill_ws", "nf4_gemm_prefill_workspace_bytes",
                     "nf4_embed",
                     "nf4_ring_create", "nf4_ring_gemm", "nf4_ring_slot_bytes", "nf4_ring_destroy",
                     "nf4_codebook", "nf4_strerror"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_codebook_bitwise_equals_oracle(lib):
    out = (ctypes.c_float * 16)()
    lib.nf4_codebook(out)
    got = np.frombuffer(bytes(out), dtype=np.float32)
    _, l32 = oracle.codebook()
    assert np.array_equal(got.view(np.uint32), l32.view(np.uint32))


P = ctypes.c_void_p(0x100000)      # fake, 16-byte aligned; never dereferenced on these paths
P_ODD = ctypes.c_void_p(0x100002)  # 2-byte aligned only
NULL = ctypes.c_void_p(0)
EINVAL, EALIGN, ERANGE = -1, -2, -3


@pytest.mark.parametrize("N,K,expect", [(0, 64, EINVAL), (-1, 64, EINVAL), (4, 0, EINVAL),
                                        (4, 100, EINVAL), (4, 65, EINVAL), (4, 32768 + 64, ERANGE),
                                        (2 ** 31, 64, ERANGE), (2 ** 17, 32768, ERANGE),
                                        (2 ** 26, 64, ERANGE)])
def test_shape_validation(lib, N, K, expect):
    assert lib.nf4_gemv(P, P, N, K, P, P, NULL) == expect
    assert lib.nf4_gemm_smallm(P, P, N, K, P, 4, P, NULL) == expect
    assert lib.nf4_gemm_prefill(P, P, N, K, P, 64, P, NULL) == expect
    assert lib.nf4_pack(P, N, K, P, P, NULL, NULL) == expect
    assert lib.nf4_unpack(P, P, N, K, P, NULL) == expect
    assert lib.nf4_embed(P, P, N, K, P, 4, P, NULL, NULL) == expect


def test_null_pointers(lib):
    assert lib.nf4_gemv(NULL, P, 4, 64, P, P, NULL) == EINVAL
    assert lib.nf4_gemv(P, NULL, 4, 64, P, P, NULL) == EINVAL
    assert lib.nf4_gemv(P, P, 4, 64, NULL, P, NULL) == EINVAL
    assert lib.nf4_gemv(P, P, 4, 64, P, NULL, NULL) == EINVAL
    assert lib.nf4_pack(NULL, 4, 64, P, P, NULL, NULL) == EINVAL
    assert lib.nf4_unpack(P, P, 4, 64, NULL, NULL) == EINVAL


@pytest.mark.parametrize("M", [0, -3, 33, 1000])
def test_m_range(lib, M):
    assert lib.nf4_gemm_smallm(P, P, 4, 64, P, M, P, NULL) == ERANGE


@pytest.mark.parametrize("M,K", [(0, 64), (-3, 64), (2 ** 24, 64), (2 ** 15, 32768)])
def test_prefill_m_range(lib, M, K):
    assert lib.nf4_gemm_prefill(P, P, 4, K, P, M, P, NULL) == ERANGE


def test_prefill_null_and_alignment(lib):
    for args in ((NULL, P, P, P), (P, NULL, P, P), (P, P, NULL, P), (P, P, P, NULL)):
        c, s, x, y = args
        assert lib.nf4_gemm_prefill(c, s, 4, 64, x, 64, y, NULL) == EINVAL
    assert lib.nf4_gemm_prefill(P_ODD, P, 4, 64, P, 64, P, NULL) == EALIGN
    assert lib.nf4_gemm_prefill(P, ctypes.c_void_p(0x100001), 4, 64, P, 64, P, NULL) == EALIGN
    assert lib.nf4_gemm_prefill(P, P, 4, 64, P_ODD, 64, P, NULL) == EALIGN
    assert lib.nf4_gemm_prefill(P, P, 4, 64, P, 64, P_ODD, NULL) == EALIGN


def test_smallm_workspace_sizes(lib):
    wb = lib.nf4_gemm_smallm_workspace_bytes
    assert wb(0, 64, 8) == -1 and wb(4, 100, 8) == -1 and wb(4, 64, 0) == -1 and wb(4, 64, 33) == -1
    assert wb(6144, 4096, 2) == 0          # vector-ALU path: never splits
    assert wb(28672, 4096, 32) == 0        # enough column tiles for every CU
    assert wb(4096, 4096, 16) > 0          # M = 9..32: the streaming form splits K in two
    assert wb(4096, 4096, 4) == 0          # M <= 8, one tile per CU: no split
    assert wb(4096, 14336, 4) == 0
    assert wb(6144, 4096, 5) > 0           # 257 to 512 tiles: streaming form, 2 splits
    assert wb(28672, 4096, 8) == 0         # ... but not over 512 tiles
    assert wb(6144, 2048, 8) == 0          # ... nor below 4096 of K
    assert wb(4096, 4096, 32) > 0          # one tile per CU at M > 16: two splits
    assert wb(6144, 4096, 32) > 0          # fewer workgroups than CUs: three tiles, two splits
    assert wb(4096, 14336, 16) > 0         # long K at M 5..16: two tiles, two splits
    assert wb(4096, 14336, 8) == 0         # M <= 8 with K % 256 == 0, one tile per CU: none
    assert wb(4096, 14464, 8) > 0          # (K = 14464: 226 groups, pair steps, split)
    assert wb(4096, 14336, 32) > 0 and wb(4096, 14336, 32) % 256 == 0
    assert wb(4096, 1024, 32) == 0         # too few pair steps to split
    assert wb(33, 320, 8) == 0


def test_smallm_ws_validation(lib):
    W = ctypes.c_void_p(0x200000)
    need = lib.nf4_gemm_smallm_workspace_bytes(4096, 14336, 32)
    # a split shape without (enough) workspace, or a misaligned one, is refused
    assert lib.nf4_gemm_smallm_ws(P, P, 4096, 14336, P, 32, P, NULL, 0, NULL) == ERANGE
    assert lib.nf4_gemm_smallm_ws(P, P, 4096, 14336, P, 32, P, W, need - 1, NULL) == ERANGE
    assert lib.nf4_gemm_smallm_ws(P, P, 4096, 14336, P, 32, P, ctypes.c_void_p(0x200010),
                                  need, NULL) == EALIGN
    assert lib.nf4_gemm_smallm_ws(P, P, 4096, 14336, P, 40, P, W, need, NULL) == ERANGE
    assert lib.nf4_gemm_smallm_ws(NULL, P, 4096, 14336, P, 32, P, W, need, NULL) == EINVAL


def test_prefill_workspace_sizes_and_validation(lib):
    wb = lib.nf4_gemm_prefill_workspace_bytes
    assert wb(0, 64, 64) == -1 and wb(4, 64, 0) == -1 and wb(4, 2 ** 15, 2 ** 15) == -1
    assert wb(4096, 4096, 512) == 0 and wb(1000, 576, 64) == 0
    need = wb(4096, 4096, 64)
    assert need > 0 and need % 256 == 0
    W = ctypes.c_void_p(0x200000)
    assert lib.nf4_gemm_prefill_ws(P, P, 4096, 4096, P, 64, P, NULL, 0, NULL) == ERANGE
    assert lib.nf4_gemm_prefill_ws(P, P, 4096, 4096, P, 64, P, W, need - 1, NULL) == ERANGE
    assert lib.nf4_gemm_prefill_ws(P, P, 4096, 4096, P, 64, P, ctypes.c_void_p(0x200010),
                                   need, NULL) == EALIGN
    assert lib.nf4_gemm_prefill_ws(P, P, 4096, 4096, P, 0, P, W, need, NULL) == ERANGE


def test_alignment(lib):
    assert lib.nf4_gemv(P_ODD, P, 4, 64, P, P, NULL) == EALIGN   # codes need 16 B
    assert lib.nf4_gemv(P, P, 4, 64, P_ODD, P, NULL) == EALIGN   # x needs 16 B
    assert lib.nf4_gemv(P, P, 4, 64, P, P_ODD, NULL) == EALIGN   # y needs 4 B
    assert lib.nf4_gemv(P, ctypes.c_void_p(0x100001), 4, 64, P, P, NULL) == EALIGN
    assert lib.nf4_unpack(P, P, 4, 64, P_ODD, NULL) == EALIGN


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.nf4_strerror(code), bytes)


def test_embed_validation(lib):
    assert lib.nf4_embed(NULL, P, 4, 64, P, 1, P, NULL, NULL) == EINVAL
    assert lib.nf4_embed(P, P, 4, 64, NULL, 1, P, NULL, NULL) == EINVAL   # ids
    assert lib.nf4_embed(P, P, 4, 64, P, 1, NULL, NULL, NULL) == EINVAL   # out
    assert lib.nf4_embed(P, P, 4, 64, P, -1, P, NULL, NULL) == EINVAL     # T < 0
    assert lib.nf4_embed(P, P, 4, 64, P, 1, P_ODD, NULL, NULL) == EALIGN  # out needs 16 B
    assert lib.nf4_embed(P, P, 4, 64, ctypes.c_void_p(0x100004), 1, P, NULL, NULL) == EALIGN
    assert lib.nf4_embed(P, P, 4, 64, P, 2 ** 31, P, NULL, NULL) == ERANGE


@pytest.mark.parametrize("K", [64, 2048, 2112, 4096, 32768])
def test_embed_row_limit_fits_one_dispatch(lib, K):
    """T beyond what one dispatch's 2^32 - 1 work-items cover is refused before
    anything is enqueued (status word included)."""
    bpr = -(-(K // 8) // 256)
    limit = 8 * (((2 ** 32 - 1) // 256) // bpr)
    # the launch grid at the limit: ceil(T / 8) blocks per row-block, 256 threads each
    assert -(-limit // 8) * bpr * 256 <= 2 ** 32 - 1
    assert lib.nf4_embed(P, P, 4, K, P, limit + 1, P, NULL, NULL) == ERANGE
    assert lib.nf4_embed(P, P, 4, K, P, limit + 1, P, P, NULL) == ERANGE


def test_ring_validation_without_a_device(lib):
    out = ctypes.c_void_p()
    assert lib.nf4_ring_create(None, P, P, 1024, NULL, NULL) == EINVAL
    assert lib.nf4_ring_create(ctypes.byref(out), NULL, P, 1024, NULL, NULL) == EINVAL
    assert lib.nf4_ring_create(ctypes.byref(out), P, P, 0, NULL, NULL) == EINVAL
    assert lib.nf4_ring_create(ctypes.byref(out), ctypes.c_void_p(0x100010), P, 1024, NULL,
                               NULL) == EALIGN
    assert lib.nf4_ring_gemm(NULL, P, P, 4, 64, P, 1, P) == EINVAL
    assert lib.nf4_ring_destroy(NULL) == EINVAL
    # codes at offset 0, scales on the next 256-byte boundary
    assert lib.nf4_ring_slot_bytes(4, 64) == 256 + 4 * 2
    assert lib.nf4_ring_slot_bytes(4096, 4096) == 4096 * 2048 + 4096 * 64 * 2
    assert lib.nf4_ring_slot_bytes(4, 65) == -1
    # beyond the product limits: refused, not computed (the arithmetic would overflow)
    assert lib.nf4_ring_slot_bytes(2 ** 61, 2 ** 61) == -1
    assert lib.nf4_ring_slot_bytes(4, 32768 + 64) == -1
    assert lib.nf4_ring_slot_bytes(2 ** 31, 64) == -1
