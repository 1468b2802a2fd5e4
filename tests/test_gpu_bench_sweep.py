"""What bench.py times, checked against the oracle: the layer sweep built by the
bench's own setup (packing, same-x fusion, activations, workspace), captured
into a HIP graph by the bench's own capture and replayed several times; after
every replay, sampled rows of every launch's output are compared with the
oracle computed from regenerated weights.  The --embed sweep likewise, bit for
bit."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def nf4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dequant_gemv_nf4_amd as m
    m._lib._load()
    return m


def _rows(N, count, seed):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set(rng.choice(N, size=min(count, N), replace=False).tolist())
                           | {0, N - 1}), np.int64)


def _reference(set_, layer, projs, K, X, rows):
    """Oracle product for rows `rows` of the launch built from `projs` (their
    rows concatenated in order), from weights regenerated with the bench's seeds."""
    Ws, r0 = [], 0
    for proj, n, _ in projs:
        sel = rows[(rows >= r0) & (rows < r0 + n)] - r0
        if sel.size:
            W = wl.weights(n, K, set_.sigma, wl.seed_for(set_.name, layer, proj, "W"), DEV)
            Ws.append(W[torch.from_numpy(sel).to(DEV)].cpu().numpy())
            del W
        r0 += n
    p, s, st = oracle.quantize_pack(np.concatenate(Ws))
    assert st == 0
    return oracle.gemm(p, s, wl.bf16_bits(X)), p, s


@pytest.mark.parametrize("set_name,M,L", [("llama2-7b", 1, 3), ("llama3.1-8b-smallm", 8, 2),
                                          ("llama3.1-8b-smallm", 32, 2)])
def test_bench_sweep_replays_match_oracle(nf4, set_name, M, L):
    set_ = wl.ALL_SETS[set_name]
    items, _, _ = bench.setup_layer_set(set_, M, L, DEV, fused=True)
    launch = bench.make_launcher(M, items, DEV)

    def sweep():
        for it in items:
            launch(it)
    g = bench.capture(torch, sweep)
    groups = wl.launch_groups(set_, fused=True)
    refs = []
    for idx, (name, N, K, codes, scales, X, Y) in enumerate(items):
        layer, (gname, projs) = divmod(idx, len(groups))[0], groups[idx % len(groups)]
        assert gname == name
        rows = _rows(N, 24, 1000 * idx + N)
        (Yr, A), p, s = _reference(set_, layer, projs, K, X, rows)
        r = torch.from_numpy(rows).to(DEV)
        assert np.array_equal(codes[r].cpu().numpy(), p), f"{name} layer {layer} codes"
        refs.append((r, Yr, A))
    for rep in range(3):
        for it in items:
            it[6].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, N, K, _, _, _, Y), (r, Yr, A) in zip(items, refs):
            got = Y[:, r].cpu().numpy().astype(np.float64)
            ok = oracle.within_tolerance(got, Yr, A)
            assert ok.all(), (f"replay {rep}: {name} {N}x{K} M={M}: {int((~ok).sum())} of "
                              f"{ok.size} outside tolerance")


def test_bench_embed_sweep_replays_match_oracle(nf4):
    T = 32
    codes, scales, K, idsets, outs = bench.setup_embed(T, DEV, R=4)
    N = codes.shape[0]

    def sweep():
        for i in range(len(idsets)):
            nf4.nf4_embed(codes, scales, K, idsets[i], outs[i])
    sweep()
    g = bench.capture(torch, sweep)
    W = wl.weights(N, K, 0.02, wl.seed_for("embed", 0, "tok", "W"), DEV)
    expected = []
    for ids in idsets:
        rows = np.unique(ids.cpu().numpy())
        p, s, st = oracle.quantize_pack(W[torch.from_numpy(rows).to(DEV)].cpu().numpy())
        assert st == 0
        e, bad = oracle.embed(p, s, np.searchsorted(rows, ids.cpu().numpy()))
        assert bad == 0
        expected.append(e)
    del W
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, expected):
            got = o.cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(got, e), f"replay {rep}"
