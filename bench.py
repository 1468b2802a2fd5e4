#!/usr/bin/env python3
"""NF4 fused dequant-GEMV benchmark on one MI355X.

A step is one decode pass over the linear layers of a model-shaped layer set:
for every layer, every projection's packed NF4 weights are multiplied with the
layer's activations, in order, on one stream.  Projections that read the same
activations (q|k|v, gate|up) run as one product over their rows concatenated
along N (free in the row-major layout); --unfused launches them one by one.
Weights are packed once before timing (the quantizer is offline work); the step
moves the packed codes and scales, the bf16 activations and the fp32 outputs.

Default workload: Llama-2-7B shapes, 32 layers of distinct seeded weights
(3.44 GB packed, well beyond the 256 MB last-level cache), M = 1.

Output: one JSON line.  value = effective HBM GB/s over the whole timed region
(algorithmic bytes / wall time, sweeps replayed from a HIP graph captured before
timing).  roofline = the dominant kernel's algorithmic GB/s from HIP events around
graph replays of that kernel's launches (per-launch duration = elapsed / launches).
cpu_baseline = the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import json
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 / bf16 matrix cores, published
METRIC = "NF4 GEMV effective HBM GB/s and % of peak at M=1; µs/layer-set (7B shapes)"
INFINITY_CACHE_BYTES = 256 << 20  # MI355X last-level (MALL) cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--set", default="llama2-7b",
                    help="layer set: llama2-7b, llama2-13b, llama2-70b, llama3.1-8b-smallm, "
                         "llama3.1-8b-prefill (use with --m 64..512), "
                         "single-4096x4096")
    ap.add_argument("--m", type=int, default=1, help="activation rows per product")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = set's)")
    ap.add_argument("--eager", action="store_true", help="time plain launches, no HIP graph")
    ap.add_argument("--unfused", action="store_true",
                    help="launch q, k, v and gate, up separately instead of per same-x group")
    ap.add_argument("--event-launches", type=int, default=64,
                    help="launches per projection for the per-kernel event timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out", default="", help="also append the JSON line to this file")
    ap.add_argument("--embed", type=int, default=0, metavar="T",
                    help="instead of the layer set: packed-embedding rows, T token ids per "
                         "call from a 32000 x 4096 (Llama-2) vocabulary matrix")
    ap.add_argument("--copyring", action="store_true",
                    help="instead of resident weights: stream the layer set's packed matrices "
                         "from pinned host memory through two device slots (CopyRing)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times): the reference "
                         "kernel whose FETCH_SIZE / WRITE_SIZE counters calibrate the HBM "
                         "byte counters, then exit")
    return ap.parse_args()


def recorded_traffic(key):
    """HBM bytes per launch measured with rocprofv3 counters for the dominant kernel,
    if the kernel sources still hash to what was profiled (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        entry = json.load(open(path))[key]
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in entry["sources"])
        if hashlib.sha256(src).hexdigest() == entry["source_sha256"]:
            return entry["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        pass
    return None


def kernel_label(M, N, K):
    """Name of the kernel a product of this shape runs, by the library's dispatch
    rule (a label for the bench line only): the vector-ALU GEMV for M <= 2 and for
    M = 3, 4 above 5120 rows; MFMA quad steps for M <= 8 when K is a multiple of
    256; MFMA pair steps up to M = 32; the prefill tiles beyond."""
    if M <= 2 or (M <= 4 and N > 5120):
        return "gemv_valu_kernel"
    if M <= 8 and K % 256 == 0:
        return "gemm_mfma_quad_kernel"
    if M <= 32:
        return "gemm_mfma_pair_kernel" if (K // 64) % 2 == 0 else "gemm_mfma_kernel"
    return "gemm_prefill_kernel"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_baseline(set_, M, seconds):
    """Time the CPU oracle (as written, single thread) on a bounded sample: the
    first 256 rows of each projection of layer 0, the same generated weights and
    activations (drawn on the host generator: timing only, not parity)."""
    import torch

    import oracle
    import workloads as wl
    rows = 256
    items = []
    for proj, N, K in set_.projections:
        n = min(rows, N)
        W = wl.weights(n, K, set_.sigma, wl.seed_for(set_.name, 0, proj, "W"))
        p, s, _ = oracle.quantize_pack(W.numpy())
        x = wl.bf16_bits(wl.activations(M, K, wl.seed_for(set_.name, 0, proj, "x")))
        items.append((p, s, x, wl.algorithmic_bytes(n, K, M)))
    nbytes = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for p, s, x, b in items:
            oracle.gemm(p, s, x)
            nbytes += b
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    del torch
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of {set_.name}, first {rows} rows of each of the "
                      f"{len(set_.projections)} projections, M={M}, {reps} passes "
                      f"in {dt:.1f} s (fp64 dequant-then-matvec, quantization untimed)",
            "host": platform.processor() or platform.machine()}


EMBED_METRIC = "NF4 packed-embedding rows (decode only the requested rows) effective GB/s"


def bench_embed(args, torch, dev):
    """Packed embedding rows: T ids per call into bf16 rows of a Llama-2-sized
    vocabulary matrix; bytes per call = the T packed rows (codes + scales), the
    ids and the bf16 output."""
    import dequant_gemv_nf4_amd as nf4
    import oracle
    import workloads as wl
    N, K, T = 32000, 4096, args.embed
    W = wl.weights(N, K, 0.02, wl.seed_for("embed", 0, "tok", "W"), dev)
    codes, scales = nf4.pack(W)
    del W
    rng = np.random.default_rng(17)
    R = 64  # distinct id sets, rotated through
    idsets = [torch.from_numpy(rng.integers(0, N, T).astype(np.int64)).to(dev) for _ in range(R)]
    outs = [torch.empty((T, K), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    def launch(i):
        nf4.nf4_embed(codes, scales, K, idsets[i % R], outs[i % R])
    for i in range(R):
        launch(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(R):
            launch(i)
    for _ in range(max(1, args.warmup)):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    us_per_call = ms * 1e3 / (args.steps * R)
    nbytes = T * (K // 2 + 2 * (K // 64)) + 8 * T + 2 * T * K
    gbs = nbytes / us_per_call / 1e3
    log(f"embed T={T}: {us_per_call:.2f} us per call, {gbs:.0f} GB/s")
    out = {"metric": EMBED_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms / args.steps, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "nf4-w/bf16-out", "data": "synthetic",
           "config": {"workload": f"packed embedding rows, {N}x{K} vocabulary, T={T} ids per call",
                      "calls_per_step": R, "timing": "hip-graph replay"},
           "us_per_call": round(us_per_call, 3),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "embed_kernel", "bytes_per_launch": nbytes,
                        "us_per_launch": round(us_per_call, 3)}}
    if not args.no_cpu_baseline:
        ids = idsets[0].cpu().numpy()
        rows = np.unique(ids)
        p = codes[torch.from_numpy(rows).to(dev)].cpu().numpy()
        sc = scales[torch.from_numpy(rows).to(dev)].cpu().numpy().view(np.uint16)
        local = np.searchsorted(rows, ids)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            oracle.embed(p, sc, local)
            reps += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{reps} calls of T={T} rows in {dt:.1f} s"}
    print(json.dumps(out), flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(json.dumps(out) + "\n")


RING_METRIC = "NF4 GEMV over packed weights streamed from pinned host memory (CopyRing), GB/s"
HOST_LINK_GBS = 64.0  # PCIe 5.0 x16, one direction, published


def bench_copyring(args, torch, dev):
    """CopyRing: every product of the layer set reads its packed matrix from
    pinned host memory through two device slots; a step is one sweep of all
    layers.  value = algorithmic bytes per step / step time (the packed bytes
    cross the host link once per step)."""
    import dequant_gemv_nf4_amd as nf4
    import workloads as wl
    set_ = wl.ALL_SETS[args.set]
    M = args.m
    L = args.layers or min(set_.layers, 8)
    groups_ = wl.launch_groups(set_, fused=not args.unfused)
    items = []
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for layer in range(L):
        for name, projs in groups_:
            K = projs[0][2]
            N = sum(n for _, n, _ in projs)
            codes, scales = nf4.empty_packed(N, K, dev)
            r0 = 0
            for proj, n, _ in projs:
                W = wl.weights(n, K, set_.sigma, wl.seed_for(set_.name, layer, proj, "W"), dev)
                nf4.nf4_pack(W, codes[r0:r0 + n], scales[r0:r0 + n], status)
                del W
                r0 += n
            hc = torch.empty(codes.shape, dtype=codes.dtype, pin_memory=True)
            hs = torch.empty(scales.shape, dtype=scales.dtype, pin_memory=True)
            hc.copy_(codes)
            hs.copy_(scales)
            del codes, scales
            X = wl.activations(M, K, wl.seed_for(set_.name, layer, name, "x"), dev)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            items.append((name, N, K, hc, hs, X, Y))
    torch.cuda.synchronize()
    slot = max(nf4.ring_slot_bytes(N, K) for _, N, K, *_ in items)
    ring = nf4.Ring(slot, dev)
    step_bytes = sum(wl.algorithmic_bytes(N, K, M) for _, N, K, *_ in items)
    packed = sum(hc.numel() + 2 * hs.numel() for _, _, _, hc, hs, _, _ in items)
    log(f"copyring: {set_.name}, {L} layers, {packed / 1e9:.2f} GB pinned, slots 2 x {slot / 1e6:.1f} MB")

    def sweep():
        for _, N, K, hc, hs, X, Y in items:
            ring.gemm(hc, hs, X, Y)
    for _ in range(args.warmup):
        sweep()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    steps = max(1, min(args.steps, 5))
    e0.record()
    for _ in range(steps):
        sweep()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    value = step_bytes / (ms / 1e3) / 1e9
    # the same bytes copied with nothing else running: the host link's rate here
    slots = ring.slots
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for i, (_, _, _, hc, hs, _, _) in enumerate(items):
        slots[i % 2][:hc.numel()].copy_(hc.view(-1), non_blocking=True)
        slots[i % 2][hc.numel():hc.numel() + 2 * hs.numel()].view(torch.int16).copy_(
            hs.view(-1), non_blocking=True)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = packed / (c0.elapsed_time(c1) / 1e3) / 1e9
    ring.close()
    log(f"copyring: {ms * 1e3:.1f} us per step, {value:.1f} GB/s; plain H2D copy of the same "
        f"bytes {copy_gbs:.1f} GB/s")
    out = {"metric": RING_METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": ("nf4-w/bf16-x/f16-dot/fp32-acc" if M < 8 else
                  "nf4-w/bf16-x/bf16-mfma/fp32-acc" if M <= nf4.MAX_M else
                  "nf4-w/bf16-x/f16-mfma/fp32-acc"), "data": "synthetic",
           "config": {"workload": f"{set_.name} layer set through CopyRing, M={M}", "layers": L,
                      "packed_gb": round(packed / 1e9, 3), "slot_mb": round(slot / 1e6, 2),
                      "timing": "eager (two streams)"},
           "h2d_copy_gbs": round(copy_gbs, 2),
           "roofline": {"bound": "host-link", "achieved": round(value, 1), "peak": HOST_LINK_GBS,
                        "unit": "GB/s", "frac": round(value / HOST_LINK_GBS, 4), "traffic": None,
                        "kernel": "CopyRing (H2D copy + gemv_valu_kernel)"}}
    print(json.dumps(out), flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(json.dumps(out) + "\n")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_gemv_nf4_amd as nf4
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.embed:
        return bench_embed(args, torch, dev)
    if args.copyring:
        return bench_copyring(args, torch, dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))
        return
    set_ = wl.ALL_SETS[args.set]
    M = args.m
    L = args.layers or set_.layers
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')}, set {set_.name}, "
        f"layers {L}, M {M}")

    # ---- setup: generate and pack every layer's weights on the GPU
    t0 = time.perf_counter()
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    st_any = torch.zeros(1, dtype=torch.int32, device=dev)
    groups_ = wl.launch_groups(set_, fused=not args.unfused)
    items = []
    for layer in range(L):
        for name, projs in groups_:
            K = projs[0][2]
            N = sum(n for _, n, _ in projs)
            codes, scales = nf4.empty_packed(N, K, dev)
            r0 = 0
            for proj, n, _ in projs:
                W = wl.weights(n, K, set_.sigma, wl.seed_for(set_.name, layer, proj, "W"), dev)
                nf4.nf4_pack(W, codes[r0:r0 + n], scales[r0:r0 + n], status)
                st_any.bitwise_or_(status)
                del W
                r0 += n
            X = wl.activations(M, K, wl.seed_for(set_.name, layer, name, "x"), dev)
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            items.append((name, N, K, codes, scales, X, Y))
    torch.cuda.synchronize()
    if int(st_any.item()) != 0:
        raise SystemExit(f"nf4_pack flagged groups: {int(st_any.item()):#x}")
    packed_bytes = sum(c.numel() + 2 * s.numel() for _, _, _, c, s, _, _ in items)
    step_bytes = sum(wl.algorithmic_bytes(N, K, M) for _, N, K, *_ in items)
    log(f"packed {packed_bytes / 1e9:.2f} GB in {time.perf_counter() - t0:.1f} s; "
        f"{step_bytes / 1e6:.2f} MB algorithmic per step")

    # one workspace for the small-batch products that split K over workgroups:
    # every launch runs on one stream after the previous, and each call leaves
    # the workspace's counters re-armed
    wsize = nf4.smallm_workspace_bytes if M <= nf4.MAX_M else nf4.prefill_workspace_bytes
    ws_bytes = max([wsize(N, K, M) for _, N, K, *_ in items]) if M > 1 else 0
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def launch(it):
        _, N, K, codes, scales, X, Y = it
        if M == 1:
            nf4.nf4_gemv(codes, scales, X, Y)
        elif M <= nf4.MAX_M:
            nf4.nf4_gemm_smallm_ws(codes, scales, X, Y, ws)
        else:
            nf4.nf4_gemm_prefill_ws(codes, scales, X, Y, ws)

    def sweep():
        for it in items:
            launch(it)

    # ---- warmup (eager), then capture one sweep into a HIP graph outside any timer
    for _ in range(args.warmup):
        sweep()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            sweep()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sweep()
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()

    # ---- timed region: K steps
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            sweep()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    value = step_bytes * args.steps / (ms_total / 1e3) / 1e9
    log(f"{args.steps} steps: {ms_per_step * 1e3:.1f} us/step (host wall {t_wall * 1e3:.1f} ms), "
        f"{value:.0f} GB/s")

    # ---- per-kernel durations: a HIP graph of R launches of one projection
    # (rotating through the layers) replayed between two HIP events on the stream
    # the kernels run on; duration = elapsed / R (graph nodes run back to back)
    per_proj = {}
    order = [name for name, _ in groups_]
    for proj in order:
        its = [it for it in items if it[0] == proj]
        # (a set with one layer repeats its matrix: enough launches that the
        # graph's own launch cost is spread thin)
        nl = max(1, args.event_launches if len(its) < 4 else min(args.event_launches, 4 * len(its)))
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            launch(its[0])
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(nl):
                launch(its[(i * 5 + 3) % len(its)])
        g.replay()
        torch.cuda.synchronize()
        us = []
        for _ in range(5):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            us.append(a.elapsed_time(b) * 1e3 / nl)
        us = np.array(us)
        _, N, K, *_ = its[0]
        per_proj[proj] = {"N": N, "K": K, "launches": nl * len(us), "us_mean": float(us.mean()),
                          "us_median": float(np.median(us)), "us_min": float(us.min()),
                          "us_max": float(us.max()), "bytes": wl.algorithmic_bytes(N, K, M)}
        log(f"  {proj:5s} {N}x{K}: {per_proj[proj]['us_mean']:.2f} us per launch, "
            f"{per_proj[proj]['bytes'] / per_proj[proj]['us_mean'] / 1e3:.0f} GB/s")
        del g

    # dominant kernel: projections sharing the kernel instance with the largest share of
    # per-step time; for M = 1 the instance is fixed by K (row units per lane)
    groups = {}
    for proj in order:
        pp = per_proj[proj]
        key = pp["K"]
        n_in_step = sum(1 for it in items if it[0] == proj)
        g = groups.setdefault(key, {"projs": [], "time": 0.0, "bytes": 0.0, "launch_us": [],
                                    "launch_bytes": []})
        g["projs"].append(proj)
        g["time"] += pp["us_mean"] * n_in_step
        g["bytes"] += pp["bytes"] * n_in_step
        g["launch_us"].append(pp["us_mean"])
        g["launch_bytes"].append(pp["bytes"])
    dom_k = max(groups, key=lambda k: groups[k]["time"])
    dom = groups[dom_k]
    # per launch: mean algorithmic bytes / mean duration over the projections it serves
    achieved = float(np.mean(dom["launch_bytes"]) / np.mean(dom["launch_us"]) / 1e3)
    kernel_sum_us = sum(per_proj[p]["us_mean"] * sum(1 for it in items if it[0] == p)
                        for p in order)
    # the dominant kernel's roofline: the HBM stream, or the matrix cores once the
    # flops per launch take longer at their peak than the bytes at theirs
    flops = float(np.mean([2.0 * M * per_proj[p]["N"] * per_proj[p]["K"] for p in dom["projs"]]))
    us_launch = float(np.mean(dom["launch_us"]))
    if flops / (MFMA_F16_PEAK_TFLOPS * 1e6) > np.mean(dom["launch_bytes"]) / (HBM_PEAK_GBS * 1e3):
        tf = flops / us_launch / 1e6
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                "flops_per_launch": flops}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    kname = " + ".join(sorted({kernel_label(M, per_proj[p]["N"], per_proj[p]["K"])
                               for p in dom["projs"]}))
    roof.update({"traffic": recorded_traffic(f"M={M} {set_.name} " + ",".join(dom["projs"])),
                 "kernel": f"{kname} (M={M}, K={dom_k})", "projections": dom["projs"],
                 "bytes_per_launch": float(np.mean(dom["launch_bytes"])),
                 "us_per_launch": round(us_launch, 3)})

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("nf4-w/bf16-x/f16-dot/fp32-acc" if M < 8 else
                  "nf4-w/bf16-x/bf16-mfma/fp32-acc" if M <= nf4.MAX_M else
                  "nf4-w/bf16-x/f16-mfma/fp32-acc"),
        "data": "synthetic",
        "config": {"workload": f"{set_.name} layer set, M={M}", "layers": L,
                   "projections": [[p, N, K] for p, N, K in set_.projections],
                   "launches": [[name, sum(n for _, n, _ in pr), pr[0][2]] for name, pr in groups_],
                   "schedule": ("one launch per projection" if args.unfused else
                                "same-x projections fused along N (q|k|v, gate|up)"),
                   "m": M, "packed_gb": round(packed_bytes / 1e9, 3),
                   "step_algorithmic_mb": round(step_bytes / 1e6, 3),
                   "timing": "hip-graph replay" if graph is not None else "eager launches",
                   "cache": ("cold: weights rotate through more than the 256 MB infinity cache"
                             if packed_bytes > INFINITY_CACHE_BYTES else
                             "warm: all weights fit the 256 MB infinity cache")},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "us_per_layer_set": round(ms_per_step * 1e3 / L, 3),
        "kernel_us_per_layer_set": round(kernel_sum_us / L, 3),
        "per_projection": per_proj,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(set_, M, args.cpu_seconds)
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
