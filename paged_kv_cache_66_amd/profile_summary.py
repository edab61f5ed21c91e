"""Summarise rocprofv3 CSV output into short text.

    python3 -m paged_kv_cache_66_amd.profile_summary stats OUT/run_kernel_stats.csv
    python3 -m paged_kv_cache_66_amd.profile_summary pmc OUT/run_counter_collection.csv

`stats` lists per-kernel call counts and durations; `pmc` averages every
collected counter per kernel over its dispatches. Kernel names are shortened
to the function name with template arguments.
"""
from __future__ import annotations

import collections
import csv
import sys


def short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "")
    n = n[5:] if n.startswith("void ") else n
    return n.split("(")[0].replace("at::native::", "")[:90]


def stats(path: str, only: str = "") -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        if only and only not in r["Name"]:
            continue
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out)


def pmc(path: str, only: str = "") -> str:
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        if only and only not in r["Kernel_Name"]:
            continue
        agg[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = ["| kernel | counter | mean per dispatch | dispatches |", "|---|---|---|---|"]
    for k, cs in agg.items():
        for c, v in sorted(cs.items()):
            out.append(f"| {k} | {c} | {sum(v) / len(v):.6g} | {len(v)} |")
    return "\n".join(out)


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    kind, path = argv[0], argv[1]
    only = argv[2] if len(argv) > 2 else ""
    print(stats(path, only) if kind == "stats" else pmc(path, only))


if __name__ == "__main__":
    main()
