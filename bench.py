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
graph replays of that kernel's launches on the launching stream (per-launch
duration = elapsed / launches).  probe = the same launches' bytes moved by a
plain streaming kernel (probe/), the floor each launch is compared with.
cpu_baseline = the CPU oracle on a bounded sample of the same workload, on one
thread and on every host core the box gives this process.
"""
import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 / bf16 matrix cores, published
METRIC = "NF4 GEMV effective HBM GB/s and % of peak at M=1; µs/layer-set (7B shapes)"
INFINITY_CACHE_BYTES = 256 << 20  # MI355X last-level (MALL) cache
CPU_THREAD_CAP = 16  # the host cores one GPU's share of the box comes with


def parse(argv=None):
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
    ap.add_argument("--event-replays", type=int, default=20,
                    help="timed replays of each per-projection graph (p10 / p90 over them)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="seconds of oracle work for each CPU baseline leg (1 thread, N threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-probe timing")
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
    return ap.parse_args(argv)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def emit(out, path):
    line = json.dumps(out)
    print(line, flush=True)
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


# ---------------------------------------------------------------- run metadata
def sources_sha256():
    from dequant_gemv_nf4_amd import build as nb
    return nb.sources_sha256()


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def host_info():
    model = None
    cpuinfo = _read("/proc/cpuinfo") or ""
    for line in cpuinfo.splitlines():
        if line.startswith("model name"):
            model = line.split(":", 1)[1].strip()
            break
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    return {"cpu_model": model or platform.processor() or platform.machine(),
            "nproc": os.cpu_count(), "cpus_usable": affinity}


def run_info(torch, dev):
    """Commit, toolchain, GPU and host identity recorded with every line.  The
    commit comes from git when the tree has it, else from the build record the
    library build wrote; sources_sha256 always describes the kernels that ran
    (and lib_built_from_these_sources says whether the built library saw the
    same sources)."""
    head = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                           text=True, timeout=10)
        if r.returncode == 0:
            head = r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    build = {}
    try:
        build = json.load(open(os.path.join(ROOT, "dequant_gemv_nf4_amd", "build_info.json")))
    except (OSError, ValueError):
        pass
    sha = sources_sha256()
    props = torch.cuda.get_device_properties(dev)
    return {"git_commit": head or build.get("git_head"),
            "git_commit_source": "git" if head else ("build record" if build else None),
            "sources_sha256": sha,
            "lib_built_from_these_sources": build.get("sources_sha256") == sha if build else None,
            "rocm_version": _read("/opt/rocm/.info/version"),
            "hip_runtime": getattr(torch.version, "hip", None), "torch": torch.__version__,
            "gpu": props.name, "gpu_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "gpu_mem_gib": round(props.total_memory / 2 ** 30, 1),
            "host": host_info()}


def pct(values, q):
    v = np.sort(np.asarray(values, dtype=np.float64))
    return float(v[min(len(v) - 1, int(q * len(v)))])


def stats(values):
    v = np.asarray(values, dtype=np.float64)
    return {"mean": float(v.mean()), "median": float(np.median(v)), "p10": pct(v, 0.1),
            "p90": pct(v, 0.9), "min": float(v.min()), "max": float(v.max()), "n": int(v.size)}


# ---------------------------------------------------------------- workload
def recorded_traffic(key):
    """HBM bytes per launch measured with rocprofv3 counters for the dominant kernel,
    if the kernel sources still hash to what was profiled (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        entry = json.load(open(path))[key]
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in entry["sources"])
        if hashlib.sha256(src).hexdigest() == entry["source_sha256"]:
            return entry["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        pass
    return None


def stream_tiles(M, N, K, workspace=True):
    """Column tiles per workgroup of the streaming MFMA form for this shape, or None
    where the library does not run it (its plan rule, mirrored for the bench line's
    labels only): K a multiple of 256 and M <= 32; given a workspace, K split over
    up to 512 tiles of 16 columns from 4096 of K (two splits at M <= 8 or up to
    4096 of K, four above; at M <= 8 only above 256 tiles), with as many tiles per
    workgroup as splits (more above 256 tiles) and at most 2 steps of 256 per wave
    above M = 8, 4 at M <= 8 (with 4, at most 5 tiles); else unsplit over more
    tiles than CUs, 2 to 8 tiles per workgroup at M <= 8, 3 to 8 above."""
    if not 1 <= M <= 32 or (K // 64) % 4 != 0 or N < 16:
        return None
    nq, tiles = K // 256, (N + 15) // 16
    nsmax = 4 if M <= 8 else 2
    if workspace and tiles <= 512 and nq >= 16 and (M > 8 or tiles > 256):
        S = 2 if M <= 8 or nq <= 16 else 4
        it = S if tiles <= 256 else -(-(tiles * S) // 256)
        ns = -(-(-(-nq // S)) // 8)
        if ns <= nsmax and it <= 8 and (ns < 4 or it <= 5):
            return it
    ns, it = -(-nq // 8), -(-tiles // 256)
    if (tiles > 256 and 1 <= ns <= nsmax and (2 if M <= 8 else 3) <= it <= 8
            and (ns < 4 or it <= 5)):
        return it
    return None


def kernel_label(M, N, K, workspace=True):
    """Name of the kernel a product of this shape runs, by the library's dispatch
    rule (a label for the bench line only): the vector-ALU GEMV for M <= 2 and for
    M = 3, 4 above 5120 rows (but M = 4 above 16384 rows where the unsplit
    streaming form takes it); the streaming MFMA form where it has a plan
    (`stream_tiles`); else quad steps for M <= 8 with K a multiple of 256, MFMA
    pair steps up to M = 32; the prefill tiles beyond."""
    it = stream_tiles(M, N, K, workspace)
    unsplit = stream_tiles(M, N, K, False)
    if (M <= 2 or (M <= 4 and N > 5120)) and not (M == 4 and N > 16384 and unsplit):
        return "gemv_valu_kernel"
    if it is not None:
        return "gemm_mfma_stream_kernel"
    if M <= 8 and K % 256 == 0:
        return "gemm_mfma_quad_kernel"
    if M <= 32:
        return "gemm_mfma_pair_kernel" if (K // 64) % 2 == 0 else "gemm_mfma_kernel"
    return "gemm_prefill_kernel"


def dtype_label(M, shapes, workspace=True):
    """The arithmetic the kernels of this M run: f16 dot products on the vector
    ALUs, f16 MFMA (the streaming form from 5 tiles per workgroup: activations in
    f16 under a per-group power-of-two shift), bf16 MFMA with hi + lo level
    halves (every other MFMA kernel), or several of these within one step."""
    kinds = set()
    for N, K in shapes:
        k = kernel_label(M, N, K, workspace)
        if k == "gemv_valu_kernel":
            kinds.add("f16-dot")
        elif k == "gemm_mfma_stream_kernel" and stream_tiles(M, N, K, workspace) >= 5:
            kinds.add("f16-mfma")
        else:
            kinds.add("bf16-mfma")
    return "nf4-w/bf16-x/" + "+".join(sorted(kinds)) + "/fp32-acc"


def setup_layer_set(set_, M, L, dev, fused=True):
    """Generate and pack every layer's weights on the GPU (one resident buffer per
    launch, same-x projections concatenated along N when `fused`), plus each
    launch's activations and output.  Returns (items, packed_bytes, step_bytes)
    with items = [(name, N, K, codes, scales, X, Y)] in launch order."""
    import torch

    import dequant_gemv_nf4_amd as nf4
    import workloads as wl
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    st_any = torch.zeros(1, dtype=torch.int32, device=dev)
    items = []
    for layer in range(L):
        for name, projs in wl.launch_groups(set_, fused=fused):
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
    packed = sum(c.numel() + 2 * s.numel() for _, _, _, c, s, _, _ in items)
    step = sum(wl.algorithmic_bytes(N, K, M) for _, N, K, *_ in items)
    return items, packed, step


def make_launcher(M, items, dev):
    """launch(item): the product of one item through the C ABI -- nf4_gemv at
    M = 1, the small-batch entry with one shared workspace up to 32 rows, the
    prefill tiles beyond.  Every launch runs on the current stream after the
    previous, and each call leaves the workspace's counters re-armed, so one
    workspace serves the whole sweep."""
    import torch

    import dequant_gemv_nf4_amd as nf4
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
    launch.workspace = ws
    return launch


def capture(torch, fn):
    """A HIP graph of fn(), captured on a side stream after one warm call there
    (capture itself is outside every timer)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, replays):
    """Per-replay milliseconds of a graph, events on the stream it runs on."""
    g.replay()
    torch.cuda.synchronize()
    ms = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return ms


def launches_for(n_items, wanted):
    # a set with one layer repeats its matrix: enough launches that the graph's
    # own launch cost is spread thin
    return max(1, wanted if n_items < 4 else min(wanted, 4 * n_items))


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(set_, M, seconds, threads=None):
    """The CPU oracle as it stands (fp64 dequant-then-matvec, quantization
    untimed) on a bounded sample: the first 256 rows of each projection of layer
    0 (weights and activations from the same generators, on the host).  One
    thread first, then `threads` threads (default: the usable host cores, at
    most 16), each calling the unchanged oracle on its own slice of the rows;
    ctypes releases the interpreter lock during each call, so the slices run in
    parallel."""
    import oracle
    import workloads as wl
    rows = 256
    items = []
    for proj, N, K in set_.projections:
        n = min(rows, N)
        W = wl.weights(n, K, set_.sigma, wl.seed_for(set_.name, 0, proj, "W"))
        p, s, _ = oracle.quantize_pack(W.numpy())
        x = wl.bf16_bits(wl.activations(M, K, wl.seed_for(set_.name, 0, proj, "x")))
        items.append((p, s, x, n, K))
    host = host_info()
    if threads is None:
        threads = max(1, min(CPU_THREAD_CAP, host["cpus_usable"] or 1))

    def run(nthreads, secs):
        slices = []
        for p, s, x, n, K in items:
            bounds = np.linspace(0, n, nthreads + 1).astype(int)
            slices.append([(p[a:b], s[a:b], x, b - a, K) for a, b in zip(bounds[:-1], bounds[1:])
                           if b > a])
        done = [0] * nthreads
        nbytes = [0] * nthreads
        stop = threading.Event()

        def worker(t):
            while True:
                for sl in slices:
                    if t < len(sl):
                        p, s, x, n, K = sl[t]
                        oracle.gemm(p, s, x)
                        nbytes[t] += wl.algorithmic_bytes(n, K, M)
                done[t] += 1
                if stop.is_set():
                    return
        ts = [threading.Thread(target=worker, args=(t,)) for t in range(nthreads)]
        t0 = time.perf_counter()
        for t in ts:
            t.start()
        time.sleep(secs)
        stop.set()
        for t in ts:
            t.join()
        dt = time.perf_counter() - t0
        return sum(nbytes) / dt / 1e9, min(done), dt

    v1, reps1, dt1 = run(1, seconds)
    vn, repsn, dtn = run(threads, seconds)
    sample = (f"layer 0 of {set_.name}, first {rows} rows of each of the {len(items)} "
              f"projections, M={M}, fp64 dequant-then-matvec (quantization untimed)")
    return {"value": round(vn, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample}; {threads} threads over row slices, {repsn}+ passes in {dtn:.1f} s",
            "one_thread": {"value": round(v1, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"{sample}; {reps1} passes in {dt1:.1f} s"},
            "host": host}


# ---------------------------------------------------------------- probe
def probe_launches(torch, per_proj_items, M, launches_wanted, replays):
    """Per launch shape: the fastest plain streaming kernel (probe/) over the same
    codes + scales bytes, writing the same M N fp32 words, timed as the products
    are (a graph of back-to-back launches rotating over the layers' buffers)."""
    import probe
    out = {}
    for proj, its in per_proj_items.items():
        _, N, K, *_ = its[0]
        nl = launches_for(len(its), launches_wanted)
        outs = torch.empty(M * N, dtype=torch.int32, device=its[0][3].device)
        best = None
        for v in range(probe.variants()):
            def fn(v=v):
                h = torch.cuda.current_stream().cuda_stream
                for i in range(nl):
                    it = its[(i * 5 + 3) % len(its)]
                    probe.stream(it[3], it[4], outs, v, h)
            g = capture(torch, fn)
            ms = time_graph(torch, g, replays)
            us = [m * 1e3 / nl for m in ms]
            med = float(np.median(us))
            if best is None or med < best["us_median"]:
                best = {"variant": v, "us_median": med, "us_p10": pct(us, 0.1),
                        "us_p90": pct(us, 0.9)}
            del g
        out[proj] = best
    return out


# ---------------------------------------------------------------- modes
EMBED_METRIC = "NF4 packed-embedding rows (decode only the requested rows) effective GB/s"


def setup_embed(T, dev, R=64, N=32000, K=4096):
    """The --embed workload: a Llama-2-sized vocabulary matrix packed on the GPU and
    R id sets of T random ids with their outputs.  Returns (codes, scales, K,
    idsets, outs)."""
    import torch

    import dequant_gemv_nf4_amd as nf4
    import workloads as wl
    W = wl.weights(N, K, 0.02, wl.seed_for("embed", 0, "tok", "W"), dev)
    codes, scales = nf4.pack(W)
    del W
    rng = np.random.default_rng(17)
    idsets = [torch.from_numpy(rng.integers(0, N, T).astype(np.int64)).to(dev) for _ in range(R)]
    outs = [torch.empty((T, K), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    return codes, scales, K, idsets, outs


def bench_embed(args, torch, dev):
    """Packed embedding rows: T ids per call into bf16 rows of a Llama-2-sized
    vocabulary matrix; bytes per call = the T packed rows (codes + scales), the
    ids and the bf16 output."""
    import dequant_gemv_nf4_amd as nf4
    import oracle
    T = args.embed
    codes, scales, K, idsets, outs = setup_embed(T, dev)
    N, R = codes.shape[0], len(idsets)

    def sweep():
        for i in range(R):
            nf4.nf4_embed(codes, scales, K, idsets[i], outs[i])
    sweep()
    g = capture(torch, sweep)
    for _ in range(max(1, args.warmup)):
        g.replay()
    torch.cuda.synchronize()
    ms_steps = time_graph(torch, g, args.steps)
    ms = float(np.sum(ms_steps))
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
           "step_ms": {k: round(v, 5) for k, v in stats(ms_steps).items()},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "embed_kernel", "bytes_per_launch": nbytes,
                        "us_per_launch": round(us_per_call, 3)},
           "run": run_info(torch, dev)}
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
                               "sample": f"{reps} calls of T={T} rows in {dt:.1f} s",
                               "host": host_info()}
    emit(out, args.out)


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
    res, packed_dev, _ = setup_layer_set(set_, M, L, dev, fused=not args.unfused)
    items = []
    for name, N, K, codes, scales, X, Y in res:
        hc = torch.empty(codes.shape, dtype=codes.dtype, pin_memory=True)
        hs = torch.empty(scales.shape, dtype=scales.dtype, pin_memory=True)
        hc.copy_(codes)
        hs.copy_(scales)
        items.append((name, N, K, hc, hs, X, Y))
    del res
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
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
           "dtype": dtype_label(M, [(N, K) for _, N, K, *_ in items]), "data": "synthetic",
           "config": {"workload": f"{set_.name} layer set through CopyRing, M={M}", "layers": L,
                      "packed_gb": round(packed / 1e9, 3), "slot_mb": round(slot / 1e6, 2),
                      "timing": "eager (two streams)"},
           "h2d_copy_gbs": round(copy_gbs, 2),
           "roofline": {"bound": "host-link", "achieved": round(value, 1), "peak": HOST_LINK_GBS,
                        "unit": "GB/s", "frac": round(value / HOST_LINK_GBS, 4), "traffic": None,
                        "kernel": "CopyRing (H2D copy + product kernel)"},
           "run": run_info(torch, dev)}
    emit(out, args.out)


def bench_layer_set(args, torch, dev):
    import workloads as wl
    set_ = wl.ALL_SETS[args.set]
    M = args.m
    L = args.layers or set_.layers
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')}, set {set_.name}, "
        f"layers {L}, M {M}")

    # ---- setup: generate and pack every layer's weights on the GPU
    t0 = time.perf_counter()
    items, packed_bytes, step_bytes = setup_layer_set(set_, M, L, dev, fused=not args.unfused)
    groups_ = wl.launch_groups(set_, fused=not args.unfused)
    log(f"packed {packed_bytes / 1e9:.2f} GB in {time.perf_counter() - t0:.1f} s; "
        f"{step_bytes / 1e6:.2f} MB algorithmic per step")
    launch = make_launcher(M, items, dev)

    def sweep():
        for it in items:
            launch(it)

    # ---- warmup (eager), then capture one sweep into a HIP graph outside any timer
    for _ in range(args.warmup):
        sweep()
    torch.cuda.synchronize()
    graph = None
    if not args.eager:
        graph = capture(torch, sweep)
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()

    # ---- timed region: K steps, an event before each step and after the last
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record()
    for k in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            sweep()
        ev[k + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = ev[0].elapsed_time(ev[-1])
    step_ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
    ms_per_step = ms_total / args.steps
    value = step_bytes * args.steps / (ms_total / 1e3) / 1e9
    log(f"{args.steps} steps: {ms_per_step * 1e3:.1f} us/step (host wall {t_wall * 1e3:.1f} ms), "
        f"{value:.0f} GB/s")

    # ---- per-kernel durations: a HIP graph of R launches of one projection
    # (rotating through the layers) replayed between two HIP events on the stream
    # the kernels run on; duration = elapsed / R (graph nodes run back to back)
    per_proj = {}
    order = [name for name, _ in groups_]
    per_proj_items = {p: [it for it in items if it[0] == p] for p in order}
    for proj in order:
        its = per_proj_items[proj]
        nl = launches_for(len(its), args.event_launches)

        def fn(its=its, nl=nl):
            for i in range(nl):
                launch(its[(i * 5 + 3) % len(its)])
        g = capture(torch, fn)
        us = [m * 1e3 / nl for m in time_graph(torch, g, args.event_replays)]
        del g
        _, N, K, *_ = its[0]
        st = stats(us)
        per_proj[proj] = {"N": N, "K": K, "launches": nl * len(us), "us_mean": st["mean"],
                          "us_median": st["median"], "us_p10": st["p10"], "us_p90": st["p90"],
                          "us_min": st["min"], "us_max": st["max"],
                          "bytes": wl.algorithmic_bytes(N, K, M),
                          "kernel": kernel_label(M, N, K)}
        per_proj[proj]["gbs"] = per_proj[proj]["bytes"] / st["mean"] / 1e3
        log(f"  {proj:7s} {N}x{K}: {st['mean']:.2f} us per launch (p10 {st['p10']:.2f}, "
            f"p90 {st['p90']:.2f}), {per_proj[proj]['gbs']:.0f} GB/s")

    # ---- the streaming floor of each launch shape
    probe_out = None
    if not args.no_probe:
        try:
            probe_out = probe_launches(torch, per_proj_items, M, args.event_launches,
                                       args.event_replays)
        except (ImportError, OSError, RuntimeError) as e:
            log(f"probe skipped: {e}")
        if probe_out:
            for proj, pr in probe_out.items():
                pp = per_proj[proj]
                pp["probe_us"] = pr["us_median"]
                pp["probe_variant"] = pr["variant"]
                pp["pct_of_probe"] = round(100.0 * pr["us_median"] / pp["us_median"], 2)
                log(f"  {proj:7s} probe {pr['us_median']:.2f} us -> kernel at "
                    f"{pp['pct_of_probe']:.1f} % of the streaming floor")

    # dominant kernel: projections sharing the kernel instance with the largest share of
    # per-step time; for M = 1 the instance is fixed by K (row units per lane)
    groups = {}
    for proj in order:
        pp = per_proj[proj]
        key = pp["K"]
        n_in_step = len(per_proj_items[proj])
        g = groups.setdefault(key, {"projs": [], "time": 0.0, "launch_us": [], "launch_bytes": []})
        g["projs"].append(proj)
        g["time"] += pp["us_mean"] * n_in_step
        g["launch_us"].append(pp["us_mean"])
        g["launch_bytes"].append(pp["bytes"])
    dom_k = max(groups, key=lambda k: groups[k]["time"])
    dom = groups[dom_k]
    achieved = float(np.mean(dom["launch_bytes"]) / np.mean(dom["launch_us"]) / 1e3)
    kernel_sum_us = sum(per_proj[p]["us_mean"] * len(per_proj_items[p]) for p in order)
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
    kname = " + ".join(sorted({per_proj[p]["kernel"] for p in dom["projs"]}))
    roof.update({"traffic": recorded_traffic(f"M={M} {set_.name} " + ",".join(dom["projs"])),
                 "kernel": f"{kname} (M={M}, K={dom_k})", "projections": dom["projs"],
                 "bytes_per_launch": float(np.mean(dom["launch_bytes"])),
                 "us_per_launch": round(us_launch, 3),
                 "us_per_launch_p10": round(float(np.mean([per_proj[p]["us_p10"]
                                                           for p in dom["projs"]])), 3),
                 "us_per_launch_p90": round(float(np.mean([per_proj[p]["us_p90"]
                                                           for p in dom["projs"]])), 3)})
    if probe_out and roof["bound"] == "hbm":
        probe_us = float(np.mean([per_proj[p]["probe_us"] for p in dom["projs"]]))
        roof["probe_us_per_launch"] = round(probe_us, 3)
        roof["pct_of_probe"] = round(100.0 * probe_us / us_launch, 2)

    shapes = [(N, K) for _, N, K, *_ in items]
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
        "dtype": dtype_label(M, shapes),
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
        "step_ms": {k: round(v, 5) for k, v in stats(step_ms).items()},
        "kernel_us_per_layer_set": round(kernel_sum_us / L, 3),
        "per_projection": per_proj,
        "roofline": roof,
        "run": run_info(torch, dev),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(set_, M, args.cpu_seconds)
    emit(out, args.out)


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_gemv_nf4_amd  # noqa: F401  (fails loudly if the library is missing)

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
    return bench_layer_set(args, torch, dev)


if __name__ == "__main__":
    main()
