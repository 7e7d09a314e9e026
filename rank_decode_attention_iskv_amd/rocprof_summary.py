"""Summaries of rocprofv3 result databases (SQLite) as short text.

    python -m rank_decode_attention_iskv_amd.rocprof_summary trace RUN_results.db [--match S ...] [--last N]
        per-kernel dispatch count and duration statistics (us); with --last N,
        over the last N dispatches of each kernel only
    python -m rank_decode_attention_iskv_amd.rocprof_summary pmc RUN_results.db [--match S ...]
        per-kernel average of every collected counter per dispatch

Kernel names are shortened (namespace and argument list dropped).
"""

from __future__ import annotations

import argparse
import re
import sqlite3
from collections import defaultdict


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("iskv::", "")
    name = re.sub(r"\(.*$", "", name)           # argument list
    name = name.replace("void ", "").replace("at::native::", "")
    return name if len(name) <= 110 else name[:107] + "..."


def _table(cur, *candidates):
    names = {r[0] for r in cur.execute("select name from sqlite_master where type in ('table','view')")}
    for c in candidates:
        if c in names:
            return c
    raise SystemExit(f"none of {candidates} in the database (tables: {sorted(names)})")


def _cols(cur, table):
    return {r[1]: i for i, r in enumerate(cur.execute(f"pragma table_info({table})"))}


def trace(db: str, match: list[str], last: int = 0) -> str:
    cur = sqlite3.connect(db).cursor()
    t = _table(cur, "kernels")
    ci = _cols(cur, t)
    name_c = "kernel_name" if "kernel_name" in ci else "name"
    stats = defaultdict(list)
    for r in sorted(cur.execute(f"select * from {t}"), key=lambda r: r[ci["start"]]):
        stats[r[ci[name_c]]].append((r[ci["end"]] - r[ci["start"]]) / 1000.0)
    if last > 0:
        stats = {k: v[-last:] for k, v in stats.items()}
    lines = [f"{'dispatches':>10} {'avg_us':>10} {'median_us':>10} {'min_us':>9} {'max_us':>9} {'total_ms':>9}  kernel"]
    for n, ds in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        s = _short(n)
        if match and not any(m in s for m in match):
            continue
        ds.sort()
        lines.append(f"{len(ds):10d} {sum(ds) / len(ds):10.2f} {ds[len(ds) // 2]:10.2f} {ds[0]:9.2f} "
                     f"{ds[-1]:9.2f} {sum(ds) / 1000:9.2f}  {s}")
    return "\n".join(lines)


def pmc(db: str, match: list[str]) -> str:
    cur = sqlite3.connect(db).cursor()
    t = _table(cur, "counters_collection")
    ci = _cols(cur, t)
    name_c = "counter_name" if "counter_name" in ci else next(c for c in ci if "name" in c and "kernel" not in c)
    val_c = "value" if "value" in ci else next(c for c in ci if "value" in c)
    kern_c = "kernel_name" if "kernel_name" in ci else None
    disp_c = "dispatch_id" if "dispatch_id" in ci else None
    if kern_c is None:
        raise SystemExit(f"no kernel name column in {t}: {sorted(ci)}")
    tot = defaultdict(float)
    disp = defaultdict(set)
    for r in cur.execute(f"select * from {t}"):
        key = (_short(r[ci[kern_c]]), r[ci[name_c]])
        tot[key] += r[ci[val_c]]
        disp[key].add(r[ci[disp_c]] if disp_c else len(disp[key]))
    lines = [f"{'dispatches':>10} {'avg_per_dispatch':>18}  counter  kernel"]
    for (k, c) in sorted(tot):
        if match and not any(m in k for m in match):
            continue
        n = max(1, len(disp[(k, c)]))
        lines.append(f"{n:10d} {tot[(k, c)] / n:18.1f}  {c}  {k}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=["trace", "pmc"])
    ap.add_argument("db")
    ap.add_argument("--match", nargs="*", default=[])
    ap.add_argument("--last", type=int, default=0)
    a = ap.parse_args()
    print(trace(a.db, a.match, a.last) if a.mode == "trace" else pmc(a.db, a.match))


if __name__ == "__main__":
    main()
