"""Summaries of rocprofv3 result databases (rocpd SQLite) for the NF4 kernels.

    python -m dequant_gemv_nf4_amd.rocpd_summary trace  <results.db> [name-filter]
    python -m dequant_gemv_nf4_amd.rocpd_summary pmc    <results.db> [name-filter]

`trace` groups dispatches by (kernel, grid, workgroup) and prints count, mean,
median, p10 and p90 duration.  `pmc` prints the mean of every collected counter
per (kernel, grid).  Both read only what rocprofv3 wrote.
"""
import collections
import sqlite3
import statistics
import sys


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")


def trace(path, filt=""):
    db = sqlite3.connect(path)
    rows = db.execute("select name, grid_x, workgroup_x, start, end from kernels order by start")
    groups = collections.OrderedDict()
    for name, gx, wx, s, e in rows:
        if filt and filt not in name:
            continue
        groups.setdefault((_short(name), gx, wx), []).append((e - s) / 1e3)
    out = []
    for (name, gx, wx), d in groups.items():
        d = sorted(d)
        out.append(f"{name:48s} grid {gx:8d} wg {wx:4d} n {len(d):5d} "
                   f"mean {statistics.mean(d):9.3f} us  median {statistics.median(d):9.3f}  "
                   f"p10 {d[len(d) // 10]:9.3f}  p90 {d[(len(d) * 9) // 10]:9.3f}")
    return out


def pmc(path, filt=""):
    db = sqlite3.connect(path)
    rows = db.execute("select kernel_name, grid_size, counter_name, value from counters_collection")
    agg = collections.OrderedDict()
    for name, grid, counter, value in rows:
        if filt and filt not in name:
            continue
        agg.setdefault((_short(name), grid), collections.defaultdict(list))[counter].append(value)
    out = []
    for (name, grid), d in agg.items():
        vals = ", ".join(f"{k}={statistics.mean(v):.1f}" for k, v in sorted(d.items()))
        out.append(f"{name:48s} grid {grid:8d} n {len(next(iter(d.values()))):4d}  {vals}")
    return out


if __name__ == "__main__":
    mode, path = sys.argv[1], sys.argv[2]
    filt = sys.argv[3] if len(sys.argv) > 3 else ""
    print("\n".join(trace(path, filt) if mode == "trace" else pmc(path, filt)))
