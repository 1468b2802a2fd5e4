"""The largest matrix one call accepts: codes of N * K / 2 bytes just below 2^31
(K = 4096 columns, N = 1048575 rows: 2 GiB of codes from 16 GiB of fp32
weights), so the 32-bit byte offsets in the kernels reach their limit and the
last tile is ragged.  Packing and embedding rows are checked bit for bit and the
products against the oracle on sampled rows, the last one included."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
K = 4096
N = (1 << 31) // (K // 2) - 1


@pytest.fixture(scope="module")
def packed():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_gemv_nf4_amd as nf4
    nf4._lib._load()
    assert N * (K // 2) < 2 ** 31 <= (N + 1) * (K // 2)
    W = wl.weights(N, K, 0.02, seed=777, device=DEV)
    codes, scales = nf4.empty_packed(N, K, DEV)
    st = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    nf4.nf4_pack(W, codes, scales, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rng = np.random.default_rng(778)
    rows = np.array(sorted(set(rng.choice(N, size=40, replace=False).tolist())
                           | {0, 1, N // 2, N - 2, N - 1}), np.int64)
    r = torch.from_numpy(rows).to(DEV)
    ref_p, ref_s, ref_st = oracle.quantize_pack(W[r].cpu().numpy())
    assert ref_st == 0
    del W
    torch.cuda.empty_cache()
    yield nf4, codes, scales, rows, r, ref_p, ref_s
    del codes, scales
    torch.cuda.empty_cache()


def test_max_size_packing(packed):
    nf4, codes, scales, rows, r, ref_p, ref_s = packed
    assert np.array_equal(codes[r].cpu().numpy(), ref_p)
    assert np.array_equal(scales[r].cpu().view(torch.int16).numpy().view(np.uint16), ref_s)


def test_max_size_embed_rows(packed):
    nf4, codes, scales, rows, r, ref_p, ref_s = packed
    got = nf4.embed(codes, scales, K, r).cpu().view(torch.int16).numpy().view(np.uint16)
    want, st = oracle.embed(ref_p, ref_s, np.arange(len(rows)))
    assert st == 0
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [1, 2, 8, 32, 64])
def test_max_size_products(packed, M):
    nf4, codes, scales, rows, r, ref_p, ref_s = packed
    X = wl.activations(M, K, seed=779 + M, device=DEV)
    Y = nf4.gemv(codes, scales, X[0]).reshape(1, -1) if M == 1 else nf4.gemm(codes, scales, X)
    torch.cuda.synchronize()
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    Ys = Y[:, r].cpu().numpy().astype(np.float64)
    ok = oracle.within_tolerance(Ys, Yr, A)
    assert ok.all(), f"M={M}: {int((~ok).sum())} of {ok.size} outside tolerance"
