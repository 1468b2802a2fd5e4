"""nf4_gemm_smallm_noalloc (the entry point that allocates nothing, its K-split
scratch a library-owned device array) against nf4_gemm_smallm_ws with a caller
workspace: the same bits, through the C ABI, on consecutive calls whose second
is smaller (so the scratch holds the previous call's partials and counters),
and within tolerance of the oracle."""
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


def _case(nf4, M, N, K, seed):
    W = wl.weights(N, K, 0.02, seed=seed, device=DEV)
    codes, scales = nf4.pack(W)
    X = wl.activations(M, K, seed=seed + 1, device=DEV)
    return W, codes, scales, X


def _with_ws(nf4, codes, scales, X):
    N, K, M = codes.shape[0], X.shape[1], X.shape[0]
    need = nf4.smallm_workspace_bytes(N, K, M)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    nf4.nf4_gemm_smallm_ws(codes, scales, X, Y, ws if need else None)
    return Y


def _oracle_check(W, X, Y, rows):
    r = torch.from_numpy(rows).to(DEV)
    p, s, _ = oracle.quantize_pack(W[r].cpu().numpy())
    Yr, A = oracle.gemm(p, s, wl.bf16_bits(X))
    ok = oracle.within_tolerance(Y[:, r].cpu().numpy().astype(np.float64), Yr, A)
    assert ok.all(), f"{int((~ok).sum())} outside tolerance"


# (M, N, K) pairs: a split call, then a smaller one (fewer splits / tiles), then
# one that does not split at all, and a vector-ALU one
SEQUENCES = [
    [(32, 4096, 14336), (32, 4096, 4096)],
    [(16, 4096, 14336), (8, 1000, 2048)],
    [(32, 6144, 4096), (24, 300, 2048), (2, 512, 1024)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "-".join(f"{m}x{n}x{k}" for m, n, k in s))
def test_noalloc_matches_the_workspace_entry_point(nf4, seq):
    assert nf4.noalloc_max_bytes() >= max(nf4.smallm_workspace_bytes(n, k, m) for m, n, k in seq)
    for i, (M, N, K) in enumerate(seq):
        W, codes, scales, X = _case(nf4, M, N, K, seed=7000 + 31 * i + N)
        ref = _with_ws(nf4, codes, scales, X)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        nf4.nf4_gemm_smallm_noalloc(codes, scales, X, Y)
        Y2 = torch.full_like(Y, float("nan"))
        nf4.nf4_gemm_smallm_noalloc(codes, scales, X, Y2)   # the counters re-armed
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), f"call {i}: M={M} N={N} K={K}"
        assert torch.equal(Y2, ref), f"repeat of call {i}"
        rows = np.unique(np.r_[np.linspace(0, N - 1, 40).astype(np.int64), N - 1])
        _oracle_check(W, X, Y, rows)


def test_noalloc_rejects_bad_arguments(nf4):
    codes, scales = nf4.empty_packed(64, 1024, DEV)
    X = torch.zeros((33, 1024), dtype=torch.bfloat16, device=DEV)
    Y = torch.empty((33, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(nf4.NF4Error):
        nf4.nf4_gemm_smallm_noalloc(codes, scales, X, Y)   # M = 33 > 32
