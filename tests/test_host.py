"""Host logic of the bench and the workload definitions (no GPU needed): the
one-GPU contract of bench.py, the recorded HBM-traffic lookup, the same-x launch
groups, the algorithmic byte count, seed separation and the CPU-baseline leg."""
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (module import runs nothing)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_recorded_traffic_follows_the_source_hash():
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    table = json.load(open(path))
    for key, entry in table.items():
        if key.startswith("_"):
            continue
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in entry["sources"])
        fresh = hashlib.sha256(src).hexdigest() == entry["source_sha256"]
        got = bench.recorded_traffic(key)
        assert got == (entry["bytes_per_launch"] if fresh else None), key
        assert entry["bytes_per_launch"] == entry["read_bytes_per_launch"] + \
            entry["write_bytes_per_launch"]
    assert bench.recorded_traffic("no such kernel") is None


def test_launch_groups_fuse_same_x_projections():
    fused = wl.launch_groups(wl.SET_7B, fused=True)
    assert [(n, sum(N for _, N, _ in p), p[0][2]) for n, p in fused] == [
        ("q|k|v", 12288, 4096), ("o", 4096, 4096), ("gate|up", 22016, 4096),
        ("down", 4096, 11008)]
    plain = wl.launch_groups(wl.SET_7B, fused=False)
    assert [n for n, _ in plain] == ["q", "k", "v", "o", "gate", "up", "down"]
    # GQA: k and v are narrower but read the same x, so they still fuse
    fused70 = wl.launch_groups(wl.SET_70B, fused=True)
    assert fused70[0][0] == "q|k|v" and sum(N for _, N, _ in fused70[0][1]) == 10240
    # every projection appears exactly once either way
    for s in wl.ALL_SETS.values():
        for f in (True, False):
            got = [p for _, grp in wl.launch_groups(s, f) for p in grp]
            assert got == list(s.projections), (s.name, f)


@pytest.mark.parametrize("N,K,M", [(4096, 4096, 1), (11008, 4096, 1), (1024, 8192, 32),
                                   (64, 64, 512)])
def test_algorithmic_bytes(N, K, M):
    # codes 4 bits, one fp16 per 64 weights, bf16 activations, fp32 outputs
    assert wl.algorithmic_bytes(N, K, M) == N * K * 17 // 32 + 2 * M * K + 4 * M * N


def test_seeds_are_distinct():
    seen = set()
    for s in wl.ALL_SETS.values():
        for layer in range(4):
            for proj, _, _ in s.projections:
                for kind in ("W", "x"):
                    seen.add(wl.seed_for(s.name, layer, proj, kind))
    n = sum(len(s.projections) for s in wl.ALL_SETS.values()) * 4 * 2
    assert len(seen) == n


def test_generators_are_seeded_and_shaped():
    a = wl.weights(3, 128, 0.02, seed=7)
    b = wl.weights(3, 128, 0.02, seed=7)
    c = wl.weights(3, 128, 0.02, seed=8)
    assert a.shape == (3, 128) and bool((a == b).all()) and not bool((a == c).all())
    x = wl.activations(2, 64, seed=9)
    assert str(x.dtype) == "torch.bfloat16" and tuple(x.shape) == (2, 64)
    assert 0.01 < float(a.std()) < 0.03


def test_cpu_baseline_leg_reports_the_contract_keys():
    out = bench.cpu_baseline(wl.SINGLE_4096, 1, 0.05, threads=3)
    assert set(out) >= {"value", "unit", "cores", "kind", "sample", "one_thread", "host"}
    assert out["kind"] == "oracle" and out["cores"] == 3 and out["value"] > 0
    assert out["one_thread"]["cores"] == 1 and out["one_thread"]["value"] > 0
    assert np.isfinite(out["value"])
    assert out["host"]["nproc"] >= 1 and out["host"]["cpu_model"]


def test_cpu_baseline_threads_default_to_the_usable_cores():
    out = bench.cpu_baseline(wl.SINGLE_4096, 1, 0.05)
    assert 1 <= out["cores"] <= bench.CPU_THREAD_CAP
    assert out["cores"] == min(bench.CPU_THREAD_CAP, bench.host_info()["cpus_usable"])


def test_stats_and_dtype_labels():
    s = bench.stats([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s["median"] == 3.0 and s["min"] == 1.0 and s["max"] == 5.0 and s["n"] == 5
    assert s["p10"] <= s["median"] <= s["p90"]
    assert bench.dtype_label(1, [(4096, 4096)]) == "nf4-w/bf16-x/f16-dot/fp32-acc"
    assert bench.dtype_label(4, [(6144, 4096), (4096, 4096)]) == \
        "nf4-w/bf16-x/bf16-mfma+f16-dot/fp32-acc"
    assert bench.dtype_label(64, [(4096, 4096)]) == "nf4-w/bf16-x/bf16-mfma/fp32-acc"
    # the 8B launches: f16 MFMA where the streaming form gets 5 or more tiles (gate|up)
    b8 = [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)]
    assert bench.dtype_label(8, b8) == "nf4-w/bf16-x/bf16-mfma+f16-mfma/fp32-acc"
    assert bench.dtype_label(4, b8) == "nf4-w/bf16-x/bf16-mfma+f16-dot+f16-mfma/fp32-acc"


@pytest.mark.parametrize("M,N,K,it", [
    # the stream kernel instances the 8B kernel traces show (<rows, steps, tiles, ...>)
    (32, 28672, 4096, 7), (32, 6144, 4096, 3), (32, 4096, 4096, 2), (32, 4096, 14336, 4),
    (4, 28672, 4096, 7), (8, 28672, 4096, 7), (8, 6144, 4096, 3),
    # no plan: one tile per CU at M <= 8 (quad steps), K not a multiple of 256, M > 32
    (8, 4096, 4096, None), (8, 4096, 14336, None), (16, 4096, 14464, None),
    (64, 28672, 4096, None)])
def test_stream_tiles_follow_the_plan_rule(M, N, K, it):
    assert bench.stream_tiles(M, N, K) == it


def test_build_record_matches_the_sources():
    from dequant_gemv_nf4_amd import build as nb
    info = json.load(open(nb.BUILD_INFO))
    assert info["sources_sha256"] == nb.sources_sha256(), "library built from other sources"


@pytest.mark.parametrize("M,N,K,name", [
    (1, 4096, 4096, "gemv_valu_kernel"), (2, 28672, 4096, "gemv_valu_kernel"),
    (4, 6144, 4096, "gemv_valu_kernel"), (4, 4096, 4096, "gemm_mfma_quad_kernel"),
    (3, 28672, 4096, "gemv_valu_kernel"), (4, 28672, 4096, "gemm_mfma_stream_kernel"),
    (4, 57344, 8192, "gemv_valu_kernel"), (8, 6144, 4096, "gemm_mfma_stream_kernel"),
    (3, 4096, 14336, "gemm_mfma_quad_kernel"), (8, 28672, 4096, "gemm_mfma_stream_kernel"),
    (8, 8192, 28672, "gemm_mfma_quad_kernel"),
    (8, 4096, 14464, "gemm_mfma_pair_kernel"), (16, 4096, 4096, "gemm_mfma_stream_kernel"),
    (16, 6144, 4096, "gemm_mfma_stream_kernel"), (16, 28672, 4096, "gemm_mfma_stream_kernel"),
    (32, 4096, 14336, "gemm_mfma_stream_kernel"), (8, 4096, 14336, "gemm_mfma_quad_kernel"),
    (32, 28672, 4096, "gemm_mfma_stream_kernel"), (32, 28672, 5120, "gemm_mfma_pair_kernel"),
    (32, 100, 320, "gemm_mfma_kernel"), (64, 4096, 4096, "gemm_prefill_kernel")])
def test_bench_kernel_label(M, N, K, name):
    """The bench line names the kernel the dispatch rule picks (vector ALU for
    M <= 2 and M = 3, 4 above 5120 rows; quad steps for M <= 8 and K % 256 == 0;
    pair steps for an even group count up to M = 32; prefill beyond)."""
    assert bench.kernel_label(M, N, K) == name


def test_rocpd_summary_splits_by_preceding_kernel(tmp_path):
    """Two shapes that share a kernel and a grid (o after q|k|v, down after
    gate|up) come apart when groups are keyed by the kernel dispatched before."""
    import sqlite3
    import rocpd_summary as rs
    db = sqlite3.connect(tmp_path / "r.db")
    db.execute("create table kernels (name text, grid_x int, workgroup_x int, start int, end int)")
    db.execute("create table counters_collection (dispatch_id int, kernel_name text, "
               "grid_size int, counter_name text, value real)")
    seq = [("A(int)", 1, 10), ("B(int)", 2, 3), ("C(int)", 3, 30), ("B(int)", 2, 5)] * 3
    t = 0
    for i, (name, grid, dur_us) in enumerate(seq):
        db.execute("insert into kernels values (?, ?, 64, ?, ?)", (name, grid, t, t + dur_us * 1000))
        db.execute("insert into counters_collection values (?, ?, ?, 'X', ?)", (i, name, grid, dur_us))
        t += dur_us * 1000 + 500
    db.commit()
    plain = rs.trace(str(tmp_path / "r.db"), "B")
    assert len(plain) == 1 and " n     6 " in plain[0]
    split = rs.trace(str(tmp_path / "r.db"), "B", True)
    assert len(split) == 2
    after_a = next(l for l in split if "after A" in l)
    after_c = next(l for l in split if "after C" in l)
    assert "mean     3.000" in after_a and "mean     5.000" in after_c
    pm = rs.pmc(str(tmp_path / "r.db"), "B", True)
    assert any("after A" in l and "X=3.0" in l for l in pm)
    assert any("after C" in l and "X=5.0" in l for l in pm)
    tot = rs.total(str(tmp_path / "r.db"), ["B(", "A("])
    assert " n     6 mean     4.000" in tot[0] and " n     3 mean    10.000" in tot[1]
    assert rs._short("void (anonymous namespace)::probe_kernel<2>(int*)") == "probe_kernel<2>"
