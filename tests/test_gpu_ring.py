"""GPU checks of CopyRing (nf4_ring_*; deep-fold README, "Method", execution-path
table and Figure 1: packed matrices kept in page-locked host memory are copied
into one of two device slots, used in turn, and multiplied there by the
unchanged kernel): every product equals the resident product bit for bit and the
oracle within tolerance, over sequences long enough to reuse both slots many
times; argument errors."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def nf4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_gemv_nf4_amd as m
    m._lib._load()
    return m


def _pinned(t):
    return t.detach().cpu().contiguous().pin_memory()


def _case(nf4, N, K, M, seed):
    W = wl.weights(N, K, 0.02, seed, device=DEV)
    codes, scales = nf4.pack(W)
    X = wl.activations(M, K, seed + 1, device=DEV)
    return codes, scales, X


def _resident(nf4, codes, scales, X):
    """The same product from resident memory through nf4_gemm_smallm (the ring
    promises its bits; the binding's gemm() may split K and group sums apart)."""
    Y = torch.empty((X.shape[0], codes.shape[0]), dtype=torch.float32, device=DEV)
    nf4.nf4_gemm_smallm(codes, scales, X, Y)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("M", [1, 4, 8])
def test_ring_matches_resident_and_oracle(nf4, M):
    shapes = [(512, 1024), (300, 4096), (1024, 512), (64, 2048), (777, 1024), (512, 1024)]
    cases = [_case(nf4, N, K, M, 100 + i) for i, (N, K) in enumerate(shapes)]
    slot = max(nf4.ring_slot_bytes(N, K) for N, K in shapes)
    ring = nf4.Ring(slot, DEV)
    outs = []
    for codes, scales, X in cases:
        Y = torch.empty((M, codes.shape[0]), dtype=torch.float32, device=DEV)
        ring.gemm(_pinned(codes), _pinned(scales), X, Y)
        outs.append(Y)
    torch.cuda.synchronize()
    ring.close()
    for (codes, scales, X), Y in zip(cases, outs):
        Yres = _resident(nf4, codes, scales, X)
        assert torch.equal(Y.view(torch.int32), Yres.view(torch.int32))
        Yr, A = oracle.gemm(codes.cpu().numpy(), scales.cpu().view(torch.int16).numpy().view(np.uint16),
                            wl.bf16_bits(X))
        assert oracle.within_tolerance(Y.cpu().numpy().astype(np.float64), Yr, A).all()


def test_ring_slot_reuse_long_sequence(nf4):
    """20 products through two slots, the compute stream slowed by large M=1
    products between small ones, so that a slot overwritten too early would show."""
    K = 4096
    cases = [_case(nf4, 4096 if i % 2 else 256, K, 1, 300 + i) for i in range(20)]
    slot = nf4.ring_slot_bytes(4096, K)
    ring = nf4.Ring(slot, DEV)
    hosts = [(_pinned(c), _pinned(s)) for c, s, _ in cases]
    outs = []
    for (hc, hs), (_, _, X) in zip(hosts, cases):
        Y = torch.empty((1, hc.shape[0]), dtype=torch.float32, device=DEV)
        ring.gemm(hc, hs, X, Y)
        outs.append(Y)
    torch.cuda.synchronize()
    ring.close()
    for (codes, scales, X), Y in zip(cases, outs):
        Yres = _resident(nf4, codes, scales, X)
        assert torch.equal(Y.view(torch.int32), Yres.view(torch.int32))


def test_ring_errors(nf4):
    codes, scales, X = _case(nf4, 256, 1024, 1, 400)
    ring = nf4.Ring(nf4.ring_slot_bytes(128, 1024), DEV)   # too small for 256 rows
    Y = torch.empty((1, 256), dtype=torch.float32, device=DEV)
    with pytest.raises(nf4.NF4Error) as e:
        ring.gemm(_pinned(codes), _pinned(scales), X, Y)
    assert e.value.status == -3
    ring.close()
    ring = nf4.Ring(nf4.ring_slot_bytes(256, 1024), DEV)
    lib = nf4._lib._load()
    import ctypes
    pageable_c = codes.cpu().contiguous()
    pageable_s = scales.cpu().contiguous()
    st = lib.nf4_ring_gemm(ring._ring, ctypes.c_void_p(pageable_c.data_ptr()),
                           ctypes.c_void_p(pageable_s.data_ptr()), 256, 1024,
                           ctypes.c_void_p(X.data_ptr()), 1, ctypes.c_void_p(Y.data_ptr()))
    assert st == -1  # pageable host memory is refused
    ring.close()
