"""Summarises a rocprofv3 results database (SQLite, rocpd schema) as text.

Kernel trace:   python -m lossless_draft_verification_02_amd.rocprof_summary trace RESULTS.db [--match k_]
Counters:       python -m lossless_draft_verification_02_amd.rocprof_summary pmc RESULTS.db [--match k_]

`trace` prints calls / mean / min / max duration and resources per kernel;
`pmc` prints the mean value of every collected counter per dispatch of each
kernel (rocprofv3 reports FETCH_SIZE and WRITE_SIZE in KiB).
"""
from __future__ import annotations

import argparse
import sqlite3
import sys


def _short(name: str, width: int = 70) -> str:
    return name if len(name) <= width else name[:width - 3] + "..."


def trace(db: str, match: str = "", top: int = 25) -> str:
    cur = sqlite3.connect(db).cursor()
    rows = cur.execute(
        "select name, count(*), avg(duration), min(duration), max(duration), sum(duration), "
        "max(vgpr_count), max(accum_vgpr_count), max(sgpr_count), max(lds_size), max(grid_x), max(workgroup_x) "
        "from kernels where name like ? group by name order by sum(duration) desc", (f"%{match}%",)).fetchall()
    out = [f"{'kernel':70s} {'calls':>6s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_ms':>9s} "
           f"{'vgpr':>5s} {'agpr':>5s} {'sgpr':>5s} {'lds':>6s} {'grid':>9s} {'wg':>5s}"]
    for r in rows[:top]:
        out.append(f"{_short(r[0]):70s} {r[1]:6d} {r[2] / 1e3:9.2f} {r[3] / 1e3:9.2f} {r[4] / 1e3:9.2f} "
                   f"{r[5] / 1e6:9.3f} {r[6]:5d} {r[7]:5d} {r[8]:5d} {r[9]:6d} {r[10]:9d} {r[11]:5d}")
    return "\n".join(out)


def pmc(db: str, match: str = "") -> str:
    cur = sqlite3.connect(db).cursor()
    cols = [d[1] for d in cur.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    val_col = "value" if "value" in cols else "counter_value"
    cnt_col = "counter_name" if "counter_name" in cols else "name"
    disp_col = "dispatch_id" if "dispatch_id" in cols else "id"
    q = (f"select {name_col}, {cnt_col}, count(distinct {disp_col}), sum({val_col}) from counters_collection "
         f"where {name_col} like ? group by {name_col}, {cnt_col} order by {name_col}")
    rows = cur.execute(q, (f"%{match}%",)).fetchall()
    out = [f"{'kernel':70s} {'counter':>14s} {'dispatches':>10s} {'mean_per_dispatch':>18s}"]
    for name, counter, n, total in rows:
        out.append(f"{_short(name):70s} {counter:>14s} {n:10d} {total / max(n, 1):18.1f}")
    return "\n".join(out)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc"])
    ap.add_argument("db")
    ap.add_argument("--match", default="")
    args = ap.parse_args(argv)
    print(trace(args.db, args.match) if args.mode == "trace" else pmc(args.db, args.match))
    return 0


if __name__ == "__main__":
    sys.exit(main())
