"""Summarises a rocprofv3 results database (SQLite, rocpd schema) as text.

Kernel trace:   python -m lossless_draft_verification_02_amd.rocprof_summary trace RESULTS.db [--match k_]
Counters:       python -m lossless_draft_verification_02_amd.rocprof_summary pmc RESULTS.db [--match k_]
Counter JSON:   python -m lossless_draft_verification_02_amd.rocprof_summary json FETCH.db --write-db WRITE.db
                    [--mfma-db MFMA.db] --match KERNEL --sources SRC... [--extra '{"workload": "..."}']

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


def _per_dispatch(db: str, match: str, counter: str):
    """Mean value per dispatch of `counter` over the kernels whose name
    contains `match` (rocprofv3 already sums the counter's instances)."""
    cur = sqlite3.connect(db).cursor()
    r = cur.execute("select count(distinct dispatch_id), sum(value) from counters_collection "
                    "where kernel_name like ? and counter_name = ?", (f"%{match}%", counter)).fetchone()
    return (r[1] / r[0]) if r and r[0] else None


def counters_json(fetch_db: str, write_db: str, match: str, sources, mfma_db=None, simds: int = 1024,
                  xcds: int = 8) -> dict:
    """HBM bytes per dispatch of the kernels matching `match`: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what the same counters read for
    torch.bitwise_not over 1 GiB of int32 in the same run (1 GiB read, 1 GiB
    written).  With `mfma_db` (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE), the
    fraction of the dispatch's active cycles the MFMA units were busy:
    busy cycles summed over `simds` SIMDs / (GRBM_GUI_ACTIVE per XCD x
    simds), GRBM_GUI_ACTIVE being summed over `xcds` XCDs."""
    import hashlib
    import json  # noqa: F401  (the caller serialises)
    copy = "bitwise_not"
    f_k, f_c = _per_dispatch(fetch_db, match, "FETCH_SIZE"), _per_dispatch(fetch_db, copy, "FETCH_SIZE")
    w_k, w_c = _per_dispatch(write_db, match, "WRITE_SIZE"), _per_dispatch(write_db, copy, "WRITE_SIZE")
    fs, ws = (1 << 30) / (f_c * 1024.0), (1 << 30) / (w_c * 1024.0)
    h = hashlib.sha256()
    for f in sources:
        with open(f, "rb") as fh:
            h.update(fh.read())
    out = {"kernel_match": match, "fetch_kib_per_dispatch": round(f_k, 1), "write_kib_per_dispatch": round(w_k, 1),
           "fetch_scale": round(fs, 6), "write_scale": round(ws, 6),
           "copy_probe": "torch.bitwise_not over 1 GiB int32 (1 GiB read + 1 GiB written per dispatch)",
           "hbm_bytes_per_launch": int(round(f_k * 1024 * fs + w_k * 1024 * ws)),
           "kernel_source_sha256": h.hexdigest()}
    if mfma_db:
        busy = _per_dispatch(mfma_db, match, "SQ_VALU_MFMA_BUSY_CYCLES")
        grbm = _per_dispatch(mfma_db, match, "GRBM_GUI_ACTIVE")
        mops = _per_dispatch(mfma_db, match, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        out.update({"mfma_busy_cycles_per_dispatch": busy, "grbm_gui_active_per_dispatch": grbm,
                    "mfma_bf16_flops_per_dispatch": None if mops is None else mops * 512,
                    "mfma_busy_frac": round(busy / ((grbm / xcds) * simds), 4)})
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc", "json"])
    ap.add_argument("db", help="results database (json mode: the FETCH_SIZE run's)")
    ap.add_argument("--match", default="")
    ap.add_argument("--write-db", help="json mode: the WRITE_SIZE run's database")
    ap.add_argument("--mfma-db", help="json mode: the MFMA counters run's database")
    ap.add_argument("--sources", nargs="*", default=[], help="json mode: kernel sources to digest")
    ap.add_argument("--extra", default="{}", help="json mode: extra fields (a JSON object)")
    args = ap.parse_args(argv)
    if args.mode == "json":
        import json
        d = counters_json(args.db, args.write_db, args.match, args.sources, args.mfma_db)
        d.update(json.loads(args.extra))
        print(json.dumps(d, indent=1))
    else:
        print(trace(args.db, args.match) if args.mode == "trace" else pmc(args.db, args.match))
    return 0


if __name__ == "__main__":
    sys.exit(main())
