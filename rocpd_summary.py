"""Summaries of rocprofv3 result databases (rocpd SQLite) for the NF4 kernels.

    python rocpd_summary.py trace  <results.db> [name-filter] [prev]
    python rocpd_summary.py pmc    <results.db> [name-filter] [prev]
    python rocpd_summary.py copies <results.db> [name-filter]
    python rocpd_summary.py total  <results.db> <name-filter> [...]

`trace` groups dispatches by (kernel, grid, workgroup) and prints count, mean,
median, p10 and p90 duration.  `pmc` prints the mean of every collected counter
per (kernel, grid).  With the word `prev`, each group is split further by the
kernel dispatched just before (labelled "after <kernel>"): two shapes that
share a kernel and a grid but follow different launches come apart.  `copies` groups memory copies by direction and size (count,
mean duration, GB/s), then reports how the copies and the filtered kernels
overlap in time: the busy time of the copy engine over the span from the first
to the last copy, and how many kernels ran while a copy was in flight.
`total` prints, for each filter, the count and mean duration of every dispatch
whose full kernel name contains it (all grids together): the figure to hold
against a bench line's per-launch mean when the projections it averages are
dispatched in equal numbers.  All read only what rocprofv3 wrote.
"""
import collections
import sqlite3
import statistics
import sys


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def trace(path, filt="", by_prev=False):
    db = sqlite3.connect(path)
    rows = db.execute("select name, grid_x, workgroup_x, start, end from kernels order by start")
    groups = collections.OrderedDict()
    prev = "-"
    for name, gx, wx, s, e in rows:
        short, before, prev = _short(name), prev, _short(name)
        if filt and filt not in name:
            continue
        key = (short + (f" after {before}" if by_prev else ""), gx, wx)
        groups.setdefault(key, []).append((e - s) / 1e3)
    out = []
    for (name, gx, wx), d in groups.items():
        d = sorted(d)
        out.append(f"{name:48s} grid {gx:8d} wg {wx:4d} n {len(d):5d} "
                   f"mean {statistics.mean(d):9.3f} us  median {statistics.median(d):9.3f}  "
                   f"p10 {d[len(d) // 10]:9.3f}  p90 {d[(len(d) * 9) // 10]:9.3f}")
    return out


def pmc(path, filt="", by_prev=False):
    db = sqlite3.connect(path)
    rows = db.execute("select dispatch_id, kernel_name, grid_size, counter_name, value "
                      "from counters_collection order by dispatch_id")
    disp = collections.OrderedDict()  # dispatch -> (kernel, grid, {counter: value})
    for did, name, grid, counter, value in rows:
        disp.setdefault(did, (_short(name), grid, collections.defaultdict(float)))[2][counter] += value
    groups = collections.OrderedDict()
    prev = "-"
    for short, grid, vals in disp.values():
        before, prev = prev, short
        if filt and filt not in short:
            continue
        key = (short + (f" after {before}" if by_prev else ""), grid)
        groups.setdefault(key, []).append(vals)
    out = []
    for (name, grid), ds in groups.items():
        vals = ", ".join(f"{c}={statistics.mean(d[c] for d in ds):.1f}" for c in sorted(ds[0]))
        out.append(f"{name:48s} grid {grid:8d} n {len(ds):4d}  {vals}")
    return out


def total(path, filters):
    db = sqlite3.connect(path)
    rows = db.execute("select name, start, end from kernels").fetchall()
    out = []
    for filt in filters:
        d = sorted((e - s) / 1e3 for name, s, e in rows if filt in name)
        if d:
            out.append(f"{filt!r:40s} n {len(d):5d} mean {statistics.mean(d):9.3f} us  "
                       f"median {statistics.median(d):9.3f}")
    return out


def copies(path, filt=""):
    db = sqlite3.connect(path)
    rows = db.execute("select name, size, start, end from memory_copies order by start").fetchall()
    kern = [(s, e) for name, s, e in db.execute("select name, start, end from kernels")
            if not filt or filt in name]
    groups = collections.OrderedDict()
    for name, size, s, e in rows:
        groups.setdefault((name, size), []).append((e - s) / 1e3)
    out = []
    for (name, size), d in groups.items():
        m = statistics.mean(d)
        out.append(f"{name:32s} size {size:11d} n {len(d):4d} mean {m:9.2f} us  "
                   f"{size / m / 1e3:7.2f} GB/s")
    if rows:
        t0, t1 = rows[0][2], max(e for *_, e in rows)
        busy, cur_s, cur_e = 0, None, None
        for *_, s, e in rows:  # union of copy intervals
            if cur_e is None or s > cur_e:
                if cur_e is not None:
                    busy += cur_e - cur_s
                cur_s, cur_e = s, e
            else:
                cur_e = max(cur_e, e)
        busy += cur_e - cur_s
        inside = [k for k in kern if k[0] >= t0 and k[1] <= t1]
        during = sum(1 for ks, ke in inside
                     if any(s < ke and e > ks for *_, s, e in rows))
        moved = sum(size for _, size, _, _ in rows)
        out.append(f"copies span {(t1 - t0) / 1e3:.1f} us, copy engine busy {busy / (t1 - t0):.1%} "
                   f"of it, {moved / ((t1 - t0) / 1e3) / 1e3:.2f} GB/s over the span; "
                   f"{during} of {len(inside)} kernels in the span ran while a copy was in flight")
    return out


if __name__ == "__main__":
    mode, path = sys.argv[1], sys.argv[2]
    filt = sys.argv[3] if len(sys.argv) > 3 else ""
    if mode == "copies":
        print("\n".join(copies(path, filt)))
    elif mode == "total":
        print("\n".join(total(path, sys.argv[3:])))
    else:
        by_prev = len(sys.argv) > 4 and sys.argv[4] == "prev"
        print("\n".join({"trace": trace, "pmc": pmc}[mode](path, filt, by_prev)))
