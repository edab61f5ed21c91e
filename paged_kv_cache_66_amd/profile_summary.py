"""Summarise rocprofv3 CSV output into short text.

    python3 -m paged_kv_cache_66_amd.profile_summary stats OUT/run_kernel_stats.csv
    python3 -m paged_kv_cache_66_amd.profile_summary pmc OUT/run_counter_collection.csv
    python3 -m paged_kv_cache_66_amd.profile_summary traffic KFETCH KWRITE CFETCH CWRITE \
        COPY_BYTES KIND NAME...

`stats` lists per-kernel call counts and durations; `pmc` averages every
collected counter per kernel over its dispatches. `traffic` turns FETCH_SIZE
and WRITE_SIZE runs (KiB per dispatch) of the kernels whose names contain one
of NAME... into HBM bytes per launch of the whole call, each counter scaled
by the ratio of known bytes to what the same counter read for a plain copy
of COPY_BYTES bytes, and stamps the result with the SHA-256 of the sources
of kernel family KIND ("decode", "prefill" or "store": srchash.kernel_sha256;
the figure is stale once one of them changes). Kernel names are shortened to the
function name with template arguments.
"""
from __future__ import annotations

import collections
import csv
import os
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


def _per_dispatch(path: str, counter: str, names) -> dict:
    """Mean counter value per kernel (shortened name) over its dispatches."""
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if names and not any(n in r["Kernel_Name"] for n in names):
            continue
        acc[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def traffic(kfetch, kwrite, cfetch, cwrite, copy_bytes, kind, names) -> dict:
    if __package__ in (None, ""):
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        from paged_kv_cache_66_amd.srchash import KERNEL_SOURCES, kernel_sha256
    else:
        from .srchash import KERNEL_SOURCES, kernel_sha256

    cf = _per_dispatch(cfetch, "FETCH_SIZE", ["copy"])
    cw = _per_dispatch(cwrite, "WRITE_SIZE", ["copy"])
    fetch_factor = copy_bytes / (max(cf.values()) * 1024)
    write_factor = copy_bytes / (max(cw.values()) * 1024)
    kf = _per_dispatch(kfetch, "FETCH_SIZE", names)
    kw = _per_dispatch(kwrite, "WRITE_SIZE", names)
    per_kernel = {k: {"fetch_bytes": kf.get(k, 0) * 1024 * fetch_factor,
                      "write_bytes": kw.get(k, 0) * 1024 * write_factor} for k in sorted(set(kf) | set(kw))}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in per_kernel.values())
    return {"bytes_per_launch": round(total), "fetch_factor": round(fetch_factor, 4),
            "write_factor": round(write_factor, 4), "per_kernel": per_kernel,
            "kernel_sha256": kernel_sha256(kind), "kernel_sources": KERNEL_SOURCES[kind]}


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    kind = argv[0]
    if kind == "traffic":
        import json
        rec = traffic(argv[1], argv[2], argv[3], argv[4], float(argv[5]), argv[6], argv[7:])
        print(json.dumps(rec, indent=1))
        return
    path = argv[1]
    only = argv[2] if len(argv) > 2 else ""
    print(stats(path, only) if kind == "stats" else pmc(path, only))


if __name__ == "__main__":
    main()
