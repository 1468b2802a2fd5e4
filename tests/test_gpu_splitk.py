"""GPU parity of the small-batch product with K split over workgroups
(nf4_gemm_smallm_ws): against the CPU oracle on the shapes where the plan
splits, bitwise repeatable across calls (the workspace counters re-arm) and
across HIP-graph replays, and within tolerance of the unsplit product."""
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


def _run_ws(nf4, codes, scales, X, ws, ws_buf=None):
    buf, Y = guard.alloc((X.shape[0], codes.shape[0]), torch.float32, DEV)
    nf4.nf4_gemm_smallm_ws(codes, scales, X, Y, ws)
    torch.cuda.synchronize()
    guard.check(buf, "smallm_ws Y")
    if ws_buf is not None:
        guard.check(ws_buf, "smallm_ws workspace")
    return Y


def _rows(N, count, seed):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set(rng.choice(N, size=min(count, N), replace=False).tolist())
                           | {0, N - 1}), np.int64)


@pytest.mark.parametrize("M,N,K", [(32, 4096, 14336), (17, 4096, 14336), (24, 4096, 8192),
                                   (32, 1000, 8192), (20, 2000, 16384), (32, 37, 8320),
                                   (8, 4096, 14336), (32, 4096, 4096), (32, 6144, 4096),
                                   (16, 1000, 2048), (16, 4096, 14336), (5, 300, 8192),
                                   (24, 5000, 2048), (32, 4100, 2048), (8, 4096, 4096),
                                   (8, 6144, 4096), (6, 8000, 4096), (7, 4200, 16384),
                                   (4, 4104, 5120)])
def test_split_matches_oracle_and_repeats(nf4, M, N, K):
    need = nf4.smallm_workspace_bytes(N, K, M)
    W = wl.weights(N, K, 0.02, seed=N + K + M, device=DEV)
    X = wl.activations(M, K, seed=3 * N + K + M, device=DEV)
    codes, scales = _pack(nf4, W)
    ws_buf, ws = guard.alloc(max(need, 256), torch.uint8, DEV, fill=0)
    ws_buf[:guard.GUARD] = guard.SENTINEL
    ws_buf[guard.GUARD + ws.numel():] = guard.SENTINEL
    Y1 = _run_ws(nf4, codes, scales, X, ws, ws_buf)
    Y2 = _run_ws(nf4, codes, scales, X, ws, ws_buf)
    Y3 = _run_ws(nf4, codes, scales, X, ws, ws_buf)
    # the same bits on every call: the counters re-arm after each one
    assert torch.equal(Y1, Y2) and torch.equal(Y1, Y3)
    rows = _rows(N, 96, M * N + K) if N * K > 4096 * 1024 else np.arange(N)
    r = torch.from_numpy(rows).to(DEV)
    ref_p, ref_s, _ = oracle.quantize_pack(W[r].cpu().numpy())
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    _check(Y1[:, r], Yr, A, f"split M={M} N={N} K={K}")
    # and the unsplit product agrees within the same tolerance
    Y0 = torch.empty_like(Y1)
    nf4.nf4_gemm_smallm(codes, scales, X, Y0)
    torch.cuda.synchronize()
    _check(Y0[:, r], Yr, A, f"unsplit M={M} N={N} K={K}")


def test_split_is_used_where_planned(nf4):
    assert nf4.smallm_workspace_bytes(4096, 14336, 32) > 0
    assert nf4.smallm_workspace_bytes(1000, 8192, 32) > 0
    assert nf4.smallm_workspace_bytes(37, 8320, 32) > 0
    assert nf4.smallm_workspace_bytes(4096, 14336, 16) > 0
    # M <= 8: the streaming form splits K over 257 to 512 column tiles from 4096
    # of K; one tile per CU runs the quad steps unsplit
    assert nf4.smallm_workspace_bytes(4096, 14336, 8) == 0
    assert nf4.smallm_workspace_bytes(4096, 4096, 8) == 0
    assert nf4.smallm_workspace_bytes(6144, 4096, 8) > 0
    assert nf4.smallm_workspace_bytes(4104, 16384, 5) > 0
    assert nf4.smallm_workspace_bytes(28672, 4096, 8) == 0
    assert nf4.smallm_workspace_bytes(6144, 2048, 8) == 0
    assert nf4.smallm_workspace_bytes(6144, 4096, 32) > 0
    assert nf4.smallm_workspace_bytes(4096, 4096, 32) > 0
    assert nf4.smallm_workspace_bytes(28672, 4096, 32) == 0


def test_gemm_binding_uses_a_kept_workspace(nf4):
    N, K, M = 4096, 14336, 32
    codes, scales = _pack(nf4, wl.weights(N, K, 0.02, seed=81, device=DEV))
    X = wl.activations(M, K, seed=82, device=DEV)
    Ya = nf4.gemm(codes, scales, X)
    Yb = nf4.gemm(codes, scales, X)
    ws = nf4.workspace_for(X.device, nf4.smallm_workspace_bytes(N, K, M))
    Yc = _run_ws(nf4, codes, scales, X, ws)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb) and torch.equal(Ya, Yc)


def test_split_in_a_hip_graph(nf4):
    """Captured once, replayed several times with eager work in between: every
    replay gives the eager bits (the counters re-arm inside the graph too)."""
    N, K, M = 4096, 14336, 32
    codes, scales = _pack(nf4, wl.weights(N, K, 0.02, seed=91, device=DEV))
    X = wl.activations(M, K, seed=92, device=DEV)
    ws = torch.zeros(nf4.smallm_workspace_bytes(N, K, M), dtype=torch.uint8, device=DEV)
    ref = _run_ws(nf4, codes, scales, X, ws)
    Y = torch.zeros_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        nf4.nf4_gemm_smallm_ws(codes, scales, X, Y, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nf4.nf4_gemm_smallm_ws(codes, scales, X, Y, ws)
    for i in range(4):
        Y.zero_()
        _ = _run_ws(nf4, codes, scales, X, ws)  # eager use of the same workspace between
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref), i


def test_one_workspace_across_shapes_and_entry_points(nf4):
    """One workspace, zero-filled once, serves split calls of different shapes and
    both entry points in turn (the counter area has a fixed place and size, and
    every call leaves it zero): each result equals a fresh-workspace call's bits."""
    cases = [("smallm", 32, 4096, 14336), ("smallm", 32, 6144, 4096), ("smallm", 32, 4096, 4096),
             ("prefill", 64, 4096, 14336), ("smallm", 16, 4096, 14336), ("prefill", 128, 2048, 4096),
             ("smallm", 24, 5000, 2048), ("smallm", 32, 4096, 14336)]
    need = max((nf4.smallm_workspace_bytes if e == "smallm" else nf4.prefill_workspace_bytes)(N, K, M)
               for e, M, N, K in cases)
    shared = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, (entry, M, N, K) in enumerate(cases):
        fn = nf4.nf4_gemm_smallm_ws if entry == "smallm" else nf4.nf4_gemm_prefill_ws
        wb = (nf4.smallm_workspace_bytes if entry == "smallm" else nf4.prefill_workspace_bytes)(N, K, M)
        assert wb > 0, (entry, M, N, K)
        W = wl.weights(N, K, 0.02, seed=500 + i, device=DEV)
        X = wl.activations(M, K, seed=600 + i, device=DEV)
        codes, scales = _pack(nf4, W)
        Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        fn(codes, scales, X, Y, shared)
        fresh = torch.zeros(wb, dtype=torch.uint8, device=DEV)
        Yf = torch.empty_like(Y)
        fn(codes, scales, X, Yf, fresh)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yf), f"{entry} M={M} N={N} K={K} on the shared workspace"
        assert int(shared[:4096].count_nonzero().item()) == 0


def test_captured_workspace_survives_a_larger_call(nf4):
    """gemm() captured in a HIP graph on a stream keeps the workspace it was
    captured with even after a larger call on the same stream replaces the
    stream's workspace: the memory is not handed out again, so replays (with
    fresh allocations filled with junk in between) still match the oracle and
    the eager bits."""
    s = torch.cuda.Stream()
    N, K, M = 4096, 4096, 32
    codes, scales = _pack(nf4, wl.weights(N, K, 0.02, seed=95, device=DEV))
    X = wl.activations(M, K, seed=96, device=DEV)
    Nb, Kb = 4096, 14336
    assert 0 < nf4.smallm_workspace_bytes(N, K, M) < nf4.smallm_workspace_bytes(Nb, Kb, M)
    cb, sb = _pack(nf4, wl.weights(Nb, Kb, 0.02, seed=97, device=DEV))
    Xb = wl.activations(M, Kb, seed=98, device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ref = nf4.gemm(codes, scales, X)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        Yg = nf4.gemm(codes, scales, X)
    with torch.cuda.stream(s):
        Ybig = nf4.gemm(cb, sb, Xb)       # replaces the stream's workspace
        junk = [torch.full((1 << 20,), -1, dtype=torch.int32, device=DEV) for _ in range(8)]
    s.synchronize()
    torch.cuda.synchronize()
    rows = _rows(N, 96, 4242)
    r = torch.from_numpy(rows).to(DEV)
    ref_p, ref_s, _ = oracle.quantize_pack(
        wl.weights(N, K, 0.02, seed=95, device=DEV)[r].cpu().numpy())
    Yr, A = oracle.gemm(ref_p, ref_s, wl.bf16_bits(X))
    for i in range(3):
        with torch.cuda.stream(s):
            Yg.zero_()
            g.replay()
        s.synchronize()
        assert torch.equal(Yg, ref), i
        _check(Yg[:, r], Yr, A, f"replay {i} after a larger call")
    rb = torch.from_numpy(_rows(Nb, 64, 4343)).to(DEV)
    pb, psb, _ = oracle.quantize_pack(wl.weights(Nb, Kb, 0.02, seed=97, device=DEV)[rb].cpu().numpy())
    Ybr, Ab = oracle.gemm(pb, psb, wl.bf16_bits(Xb))
    _check(Ybig[:, rb], Ybr, Ab, "the larger call")
    del junk
