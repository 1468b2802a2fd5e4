"""GPU parity of the prefill product (nf4_gemm_prefill, 32 x 32 x 16 f16 MFMA
tiles) against the CPU oracle: Y = X . dequant(codes, scales)^T for batches
beyond 32 rows, every workgroup tile shape, ragged M and N, odd group counts,
and the exact identities of the product.  Bar: |y - y_ref| <= 2e-3 * sum_k
|w~ x| + 1e-5 per element, y_ref and the bound from oracle/ on host copies of
the generated inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

import gpu_guard as guard

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def nf4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_gemv_nf4_amd as m
    m._lib._load()  # fail loudly if the library is missing
    return m


def _pack(nf4, W):
    codes, scales = nf4.empty_packed(W.shape[0], W.shape[1], W.device)
    st = torch.zeros(1, dtype=torch.int32, device=W.device)
    nf4.nf4_pack(W, codes, scales, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return codes, scales


def _prefill(nf4, codes, scales, X):
    buf, Y = guard.alloc((X.shape[0], codes.shape[0]), torch.float32, X.device)
    nf4.nf4_gemm_prefill(codes, scales, X, Y)
    torch.cuda.synchronize()
    guard.check(buf, "prefill Y")
    return Y


def _check(Y, Yr, A, what):
    Y = Y.detach().cpu().numpy().astype(np.float64).reshape(Yr.shape)
    ok = oracle.within_tolerance(Y, Yr, A)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        det = [(tuple(i), Y[tuple(i)], Yr[tuple(i)], A[tuple(i)]) for i in idx]
        pytest.fail(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance, e.g. {det}")


def _case(nf4, M, N, K, seed, rows=None, sigma=0.02):
    """Full check (rows=None) or a check of the sampled weight rows `rows`."""
    W = wl.weights(N, K, sigma, seed=seed * 1009 + N * 31 + K, device=DEV)
    X = wl.activations(M, K, seed=seed * 2003 + M * 17 + K, device=DEV)
    codes, scales = _pack(nf4, W)
    Y = _prefill(nf4, codes, scales, X)
    if rows is None:
        ref_p, ref_s, _ = oracle.quantize_pack(W.cpu().numpy())
        Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
        _check(Y, Yr, A, f"M={M} N={N} K={K}")
    else:
        r = torch.from_numpy(rows).to(DEV)
        ref_p, ref_s, _ = oracle.quantize_pack(W[r].cpu().numpy())
        Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
        _check(Y[:, r], Yr, A, f"M={M} N={N} K={K} (sampled rows)")
    return codes, scales, X, Y


def _rows(N, count, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(N, size=min(count, N), replace=False).tolist()) | {0, N - 1}
    return np.array(sorted(rows), np.int64)


@pytest.mark.parametrize("M", [1, 7, 31, 33, 63, 64, 65, 100, 128, 129, 200, 256])
def test_prefill_m_sweep(nf4, M):
    _case(nf4, M, 272, 1024, seed=M)


@pytest.mark.parametrize("M,N,K", [(48, 33, 64), (64, 1, 128), (96, 4111, 192), (130, 300, 14336),
                                   (40, 200, 20480), (70, 129, 320), (257, 64, 2048)])
def test_prefill_shapes(nf4, M, N, K):
    _case(nf4, M, N, K, seed=11)


# workgroup tile shapes: 64 x 64 above; 64 x 128 and 128 x 128 need grids of at
# least 256 workgroups of that tile, checked on sampled weight rows
@pytest.mark.parametrize("M,N,K", [(512, 4096, 128), (256, 16384, 128), (520, 16390, 192)])
def test_prefill_large_tiles(nf4, M, N, K):
    _case(nf4, M, N, K, seed=12, rows=_rows(N, 64, M + N))


def test_prefill_exact_identities(nf4):
    N, K = 300, 1024
    W = wl.weights(N, K, 0.02, seed=5, device=DEV)
    codes, scales = _pack(nf4, W)
    for M in (33, 64, 200):
        X = wl.activations(M, K, seed=6, device=DEV)
        Y = _prefill(nf4, codes, scales, X)
        Z = _prefill(nf4, codes, scales, torch.zeros_like(X))
        Y4 = _prefill(nf4, codes, scales, (X.float() * 4.0).to(torch.bfloat16))
        Yq = _prefill(nf4, codes, scales, (X.float() * 0.25).to(torch.bfloat16))
        Y2 = _prefill(nf4, codes, scales, X)
        assert torch.all(Z == 0), M
        assert torch.equal(Y4, Y * 4.0), M
        assert torch.equal(Yq, Y * 0.25), M
        assert torch.equal(Y2, Y), M
    zc = torch.full_like(codes, 0x77)
    assert torch.all(_prefill(nf4, zc, scales, wl.activations(70, K, seed=7, device=DEV)) == 0)


def test_prefill_rows_are_independent(nf4):
    """Row m of a batch equals the same activation row computed alone (each
    row's scaling and sums depend on that row only): bitwise."""
    N, K = 200, 2048
    codes, scales = _pack(nf4, wl.weights(N, K, 0.02, seed=21, device=DEV))
    X = wl.activations(96, K, seed=22, device=DEV)
    Y = _prefill(nf4, codes, scales, X)
    for m in (0, 31, 64, 95):
        assert torch.equal(_prefill(nf4, codes, scales, X[m:m + 1].contiguous())[0], Y[m]), m


def test_prefill_activation_range_extremes(nf4):
    N, K = 64, 2048
    W = wl.weights(N, K, 0.02, seed=8, device=DEV)
    codes, scales = _pack(nf4, W)
    ref_p, ref_s, _ = oracle.quantize_pack(W.cpu().numpy())
    X = wl.activations(72, K, seed=9, device=DEV).float()
    X[0] *= 1e30
    X[1] *= 1e-30
    X[2, ::2] *= 1e6
    X[40:44] *= 3e4  # beyond the f16 range before scaling
    Xb = X.to(torch.bfloat16)
    Y = _prefill(nf4, codes, scales, Xb)
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(Xb))
    _check(Y, Yr, A, "prefill activation range")


def test_prefill_scales_only_2_byte_aligned(nf4):
    N, K, M = 96, 1024, 80
    W = wl.weights(N, K, 0.02, seed=61, device=DEV)
    codes, scales = _pack(nf4, W)
    buf = torch.zeros(N * (K // 64) + 1, dtype=torch.int16, device=DEV)
    buf[1:].copy_(scales.view(-1))
    sc = buf[1:].view(N, K // 64)
    assert sc.data_ptr() % 4 == 2
    X = wl.activations(M, K, seed=71, device=DEV)
    Y = _prefill(nf4, codes, sc, X)
    ref_p, ref_s, _ = oracle.quantize_pack(W.cpu().numpy())
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    _check(Y, Yr, A, "prefill, 2-byte aligned scales")


def test_gemm_dispatches_beyond_32_rows(nf4):
    """nf4.gemm routes M > 32 to the prefill tiles (with a kept workspace where
    the grid splits K): the same bits as the direct calls."""
    N, K = 128, 512
    codes, scales = _pack(nf4, wl.weights(N, K, 0.02, seed=31, device=DEV))
    X = wl.activations(48, K, seed=32, device=DEV)
    need = nf4.prefill_workspace_bytes(N, K, 48)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    Y = nf4.gemm(codes, scales, X)
    torch.cuda.synchronize()
    assert torch.equal(Y, _prefill_ws(nf4, codes, scales, X, ws if need else None))


@pytest.mark.parametrize("M", [64, 512])
def test_prefill_full_size_8b(nf4, M):
    """The 8B layer shapes at prefill batch sizes, sampled weight rows."""
    set_ = wl.SET_8B_SMALLM
    seen = set()
    for fused in (False, True):
        for name, projs in wl.launch_groups(set_, fused):
            N, K = sum(n for _, n, _ in projs), projs[0][2]
            if (N, K) in seen:
                continue
            seen.add((N, K))
            _case(nf4, M, N, K, seed=wl.seed_for(set_.name, 0, name, "W") % 100000,
                  rows=_rows(N, 32, N + K + M))


# ------------------------------------------------------------------ workgroup K-splits
def _prefill_ws(nf4, codes, scales, X, ws, ws_buf=None):
    buf, Y = guard.alloc((X.shape[0], codes.shape[0]), torch.float32, X.device)
    nf4.nf4_gemm_prefill_ws(codes, scales, X, Y, ws)
    torch.cuda.synchronize()
    guard.check(buf, "prefill_ws Y")
    if ws_buf is not None:
        guard.check(ws_buf, "prefill_ws workspace")
    return Y


@pytest.mark.parametrize("M,N,K", [(64, 4096, 4096), (100, 300, 2048), (70, 129, 8192),
                                   (33, 64, 4160), (128, 6144, 4096), (64, 1000, 576)])
def test_prefill_split_matches_oracle_and_repeats(nf4, M, N, K):
    need = nf4.prefill_workspace_bytes(N, K, M)
    W = wl.weights(N, K, 0.02, seed=N * 3 + K + M, device=DEV)
    X = wl.activations(M, K, seed=N + K * 5 + M, device=DEV)
    codes, scales = _pack(nf4, W)
    ws_buf, ws = guard.alloc(max(need, 256), torch.uint8, DEV, fill=0)
    ws_buf[:guard.GUARD] = guard.SENTINEL
    ws_buf[guard.GUARD + ws.numel():] = guard.SENTINEL
    Y1 = _prefill_ws(nf4, codes, scales, X, ws, ws_buf)
    Y2 = _prefill_ws(nf4, codes, scales, X, ws, ws_buf)
    Y3 = _prefill_ws(nf4, codes, scales, X, ws, ws_buf)
    # the same bits on every call: the counters re-arm after each one
    assert torch.equal(Y1, Y2) and torch.equal(Y1, Y3)
    rows = _rows(N, 64, M + N) if N * K > 2 ** 22 else np.arange(N)
    r = torch.from_numpy(rows).to(DEV)
    ref_p, ref_s, _ = oracle.quantize_pack(W[r].cpu().numpy())
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    _check(Y1[:, r], Yr, A, f"prefill split M={M} N={N} K={K}")
    Y0 = _prefill(nf4, codes, scales, X)
    _check(Y0[:, r], Yr, A, f"prefill unsplit M={M} N={N} K={K}")


# the 16-byte scale blocks (whole blocks of 8 x KS groups per workgroup, each
# in-workgroup split a contiguous KS-th of its range): 64 x 64 tiles (KS = 4),
# 64 x 128 and 128 x 128 (KS = 2), unsplit and with workgroup K-splits
@pytest.mark.parametrize("M,N,K,ws", [(64, 300, 2048, False), (100, 4096, 4096, True),
                                      (128, 11520, 1024, False), (256, 11520, 2048, False),
                                      (512, 4096, 8192, True)])
def test_prefill_scale_blocks(nf4, M, N, K, ws):
    W = wl.weights(N, K, 0.02, seed=N + 7 * K + M, device=DEV)
    X = wl.activations(M, K, seed=3 * N + K + M, device=DEV)
    codes, scales = _pack(nf4, W)
    if ws:
        need = nf4.prefill_workspace_bytes(N, K, M)
        assert need > 0
        ws_buf, w = guard.alloc(need, torch.uint8, DEV, fill=0)
        ws_buf[:guard.GUARD] = guard.SENTINEL
        ws_buf[guard.GUARD + w.numel():] = guard.SENTINEL
        Y = _prefill_ws(nf4, codes, scales, X, w, ws_buf)
    else:
        Y = _prefill(nf4, codes, scales, X)
    rows = _rows(N, 64, M + N) if N * K > 2 ** 22 else np.arange(N)
    r = torch.from_numpy(rows).to(DEV)
    ref_p, ref_s, _ = oracle.quantize_pack(W[r].cpu().numpy())
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    _check(Y[:, r], Yr, A, f"prefill scale blocks M={M} N={N} K={K} ws={ws}")


def test_prefill_split_planned_for_small_grids(nf4):
    assert nf4.prefill_workspace_bytes(4096, 4096, 64) > 0
    assert nf4.prefill_workspace_bytes(300, 2048, 100) > 0
    assert nf4.prefill_workspace_bytes(1000, 576, 64) == 0      # too few groups to split
    assert nf4.prefill_workspace_bytes(28672, 4096, 64) == 0    # grid already fills the CUs
    assert nf4.prefill_workspace_bytes(4096, 4096, 512) == 0


def test_prefill_split_in_a_hip_graph(nf4):
    N, K, M = 4096, 4096, 64
    codes, scales = _pack(nf4, wl.weights(N, K, 0.02, seed=95, device=DEV))
    X = wl.activations(M, K, seed=96, device=DEV)
    ws = torch.zeros(nf4.prefill_workspace_bytes(N, K, M), dtype=torch.uint8, device=DEV)
    ref = _prefill_ws(nf4, codes, scales, X, ws)
    Y = torch.zeros_like(ref)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        nf4.nf4_gemm_prefill_ws(codes, scales, X, Y, ws)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nf4.nf4_gemm_prefill_ws(codes, scales, X, Y, ws)
    for i in range(4):
        Y.zero_()
        _ = _prefill_ws(nf4, codes, scales, X, ws)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), i
