"""GPU parity on seeded random shapes, so that no dispatch rule or plan is only
ever run on the hand-picked shapes: every product kernel (vector-ALU GEMV, quad,
pair and one-group MFMA steps, the streaming form with and without K-splits,
the prefill tiles) gets shapes drawn from its own range, through the dispatching
entry points with and without a workspace, each checked against the CPU oracle
(all rows of the small ones, sampled rows of the large ones)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

import gpu_guard as guard

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _shapes():
    rng = np.random.default_rng(20261203)
    out = []
    for _ in range(12):   # small: every M up to 40, any K multiple of 64, ragged N
        out.append(("small", int(rng.integers(1, 41)), int(rng.integers(1, 701)),
                    64 * int(rng.integers(1, 41))))
    for _ in range(6):    # the vector-ALU GEMV: M <= 4 on more than 5120 rows
        out.append(("gemv", int(rng.integers(1, 5)), int(rng.integers(5121, 12001)),
                    64 * int(rng.integers(1, 81))))
    for _ in range(8):    # two or more column tiles per CU, K a multiple of 256: the streaming
        M = int(rng.integers(2, 33))  # form (three or more tiles above M = 8)
        out.append(("wide", M, int(rng.integers(4097, 9001) if M <= 8 else rng.integers(12289, 20001)),
                    256 * int(rng.integers(4, 21))))
    for _ in range(4):    # quad steps: M 3..8 on up to 256 column tiles, K a multiple of 256
        out.append(("quad", int(rng.integers(3, 9)), int(rng.integers(16, 4097)),
                    256 * int(rng.integers(1, 41))))
    for _ in range(6):    # long K at M 9..32: workgroup K-splits
        out.append(("longk", int(rng.integers(9, 33)), int(rng.integers(64, 3001)),
                    256 * int(rng.integers(16, 41))))
    for _ in range(6):    # prefill tiles
        out.append(("prefill", int(rng.integers(33, 201)), int(rng.integers(100, 3001)),
                    64 * int(rng.integers(1, 65))))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module")
def nf4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_gemv_nf4_amd as m
    m._lib._load()
    return m


def _pack(nf4, W):
    codes, scales = nf4.empty_packed(W.shape[0], W.shape[1], W.device)
    st = torch.zeros(1, dtype=torch.int32, device=W.device)
    nf4.nf4_pack(W, codes, scales, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return codes, scales


def _check(Y, Yr, A, what):
    Y = Y.detach().cpu().numpy().astype(np.float64).reshape(Yr.shape)
    ok = oracle.within_tolerance(Y, Yr, A)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        pytest.fail(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance, e.g. "
                    f"{[(tuple(i), Y[tuple(i)], Yr[tuple(i)]) for i in idx]}")


@pytest.mark.parametrize("kind,M,N,K", SHAPES,
                         ids=[f"{k}-M{m}-N{n}-K{kk}" for k, m, n, kk in SHAPES])
def test_random_shape_matches_oracle(nf4, kind, M, N, K):
    W = wl.weights(N, K, 0.02, seed=7 * N + 3 * K + M, device=DEV)
    X = wl.activations(M, K, seed=N + 5 * K + 11 * M, device=DEV)
    codes, scales = _pack(nf4, W)
    if N * K * M > 2 ** 27:
        rng = np.random.default_rng(N + K + M)
        rows = np.array(sorted(set(rng.choice(N, size=64, replace=False).tolist()) | {0, N - 1}))
    else:
        rows = np.arange(N)
    r = torch.from_numpy(rows).to(DEV)
    ref_p, ref_s, _ = oracle.quantize_pack(W[r].cpu().numpy())
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    what = f"{kind} M={M} N={N} K={K}"
    # the dispatching entry point (a kept workspace where the plan splits K)
    Y = nf4.gemm(codes, scales, X)
    torch.cuda.synchronize()
    _check(Y[:, r], Yr, A, what + " (gemm)")
    if M <= 32:
        # the entry point without a workspace, into a guarded output
        buf, Y0 = guard.alloc((M, N), torch.float32, DEV)
        nf4.nf4_gemm_smallm(codes, scales, X, Y0)
        torch.cuda.synchronize()
        guard.check(buf, "smallm Y")
        _check(Y0[:, r], Yr, A, what + " (smallm, no workspace)")
    else:
        buf, Y0 = guard.alloc((M, N), torch.float32, DEV)
        nf4.nf4_gemm_prefill(codes, scales, X, Y0)
        torch.cuda.synchronize()
        guard.check(buf, "prefill Y")
        _check(Y0[:, r], Yr, A, what + " (prefill, no workspace)")
