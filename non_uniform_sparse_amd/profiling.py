"""Summaries of rocprofv3 output (rocpd SQLite databases) for profiles/.

    python -m non_uniform_sparse_amd.profiling trace DIR --cmd "..." --out FILE
    python -m non_uniform_sparse_amd.profiling pmc DIR [DIR ...] --cmd "..." --out FILE
    python -m non_uniform_sparse_amd.profiling traffic --workload W --fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --out FILE

``traffic`` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the split-K
decode kernel (and, alongside, the combine) into bytes per launch, each
counter scaled by what it reads for a plain device copy of known size (1 GiB
read + 1 GiB written), and tags the record with a hash of the decode source
so stale records are ignored.
"""

from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import re
import sqlite3
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_common.h", "kvs_device.h", "kvs_internal.h"):
        h.update(open(os.path.join(PKG, "csrc", f), "rb").read())
    return h.hexdigest()


def _db(path: str) -> sqlite3.Connection:
    if path.endswith(".db"):
        return sqlite3.connect(path)
    return sqlite3.connect(glob.glob(os.path.join(path, "**", "*.db"), recursive=True)[0])


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return re.sub(r"\((kvs::|float|unsigned|int|const|at::).*$", "", name).strip()


def _grid_col(cols):
    for c in cols:
        lc = c.lower()
        if "grid" in lc and (lc.endswith("x") or lc == "grid_size"):
            return cols.index(c)
    return None


def kernel_stats(path: str) -> dict:
    """Durations (us) per (kernel, grid size): launches of one kernel at
    different sizes, e.g. whole-batch and micro-batch launches, stay apart."""
    con = _db(path)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    ki = cols.index("name") if "name" in cols else cols.index("kernel_name")
    st, en = cols.index("start"), cols.index("end")
    gi = _grid_col(cols)
    agg = collections.defaultdict(list)
    for r in con.execute("select * from kernels"):
        agg[(_short(r[ki]), r[gi] if gi is not None else "")].append((r[en] - r[st]) / 1e3)
    # a kernel launched at many sizes (one per layer, say) gets one row
    grids = collections.Counter(name for name, _ in agg)
    out = collections.defaultdict(list)
    for (name, grid), v in agg.items():
        out[(name, "various" if grids[name] > 4 else grid)].extend(v)
    return out


def pmc_stats(path: str) -> dict:
    con = _db(path)
    cols = [r[1] for r in con.execute("pragma table_info(counters_collection)")]
    ki, ci, vi = cols.index("kernel_name"), cols.index("counter_name"), cols.index("value")
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in con.execute("select * from counters_collection"):
        agg[_short(r[ki])][r[ci]].append(r[vi])
    return agg


def _header(cmd: str) -> str:
    return f"# command (run from /tmp with TMPDIR=/tmp):\n#   {cmd}\n"


def write_trace(path: str, cmd: str, out: str, pattern: str = "kvs") -> None:
    stats = kernel_stats(path)
    lines = [_header(cmd), f"{'kernel':56s} {'grid':>9s} {'calls':>6s} {'avg_us':>9s} "
             f"{'min_us':>9s} {'max_us':>9s} {'total_ms':>9s}"]
    for (name, grid), v in sorted(stats.items(), key=lambda x: -sum(x[1])):
        if pattern and not re.search(pattern, name):
            continue
        lines.append(f"{name[:56]:56s} {str(grid):>9s} {len(v):6d} {statistics.mean(v):9.2f} "
                     f"{min(v):9.2f} {max(v):9.2f} {sum(v) / 1e3:9.2f}")
    open(out, "w").write("\n".join(lines) + "\n")


def write_pmc(paths, cmd: str, out: str, pattern: str = "") -> None:
    lines = [_header(cmd)]
    for p in paths:
        lines.append(f"## {os.path.basename(p.rstrip('/'))}")
        for name, cs in pmc_stats(p).items():
            if pattern and not re.search(pattern, name):
                continue
            vals = ", ".join(f"{k}={statistics.mean(v):.6g}" for k, v in sorted(cs.items()))
            lines.append(f"{name[:64]:64s} dispatches={len(next(iter(cs.values())))} {vals}")
    open(out, "w").write("\n".join(lines) + "\n")


def _counter(path, counter, pattern):
    vals = []
    for name, cs in pmc_stats(path).items():
        if re.search(pattern, name) and counter in cs:
            vals.append(statistics.mean(cs[counter]))
    return sum(vals)


def write_traffic(workload, fetch, write, copy_fetch, copy_write, out, cmd) -> dict:
    kib = 1024.0
    # only the copy kernel: the probe's source fill writes 1 GiB too
    cf = _counter(copy_fetch, "FETCH_SIZE", r"copy") * kib
    cw = _counter(copy_write, "WRITE_SIZE", r"copy") * kib
    fs, ws = COPY_BYTES / cf, COPY_BYTES / cw
    f = _counter(fetch, "FETCH_SIZE", r"decode_kernel") * kib * fs
    w = _counter(write, "WRITE_SIZE", r"decode_kernel") * kib * ws
    cf_ = _counter(fetch, "FETCH_SIZE", r"combine_kernel") * kib * fs
    cw_ = _counter(write, "WRITE_SIZE", r"combine_kernel") * kib * ws
    rec = {"workload": workload, "kernel": "decode_kernel (the split-K decode)",
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
           "fetch_bytes_per_launch": int(f), "write_bytes_per_launch": int(w),
           "traffic_bytes_per_launch": int(f + w),
           "combine_kernel": {"fetch_bytes_per_launch": int(cf_),
                              "write_bytes_per_launch": int(cw_)},
           "source_sha256": decode_source_hash(), "commands": cmd}
    json.dump(rec, open(out, "w"), indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc", "traffic"])
    ap.add_argument("dirs", nargs="*")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--out", required=True)
    ap.add_argument("--pattern", default="kvs")
    ap.add_argument("--workload")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    a = ap.parse_args()
    if a.mode == "trace":
        write_trace(a.dirs[0], a.cmd, a.out, a.pattern)
    elif a.mode == "pmc":
        write_pmc(a.dirs, a.cmd, a.out, a.pattern)
    else:
        print(write_traffic(a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write, a.out, a.cmd))


if __name__ == "__main__":
    main()
