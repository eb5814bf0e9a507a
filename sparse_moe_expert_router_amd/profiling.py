"""Summaries of rocprofv3 output for this library's kernels (no GPU needed to run these).

Kernel statistics come from ``rocprofv3 --kernel-trace --stats --output-format csv`` (the
``*_kernel_stats.csv`` file); HBM traffic comes from two counter runs, ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` (``*_counter_collection.csv``), each in KiB per dispatch.  The counters are
scaled by what they read for a plain copy of known size (``bench.py --copy-calibration``): the
copy's bytes divided by its counter reading.

``python -m sparse_moe_expert_router_amd.profiling stats <kernel_stats.csv>`` prints a table;
``... counters <counter_collection.csv> <COUNTER>`` prints the per-kernel mean of one counter.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


def source_hash() -> str:
    """sha256 over the HIP sources, so a stored counter reading can be matched to the code."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, name), "rb") as fh:
                h.update(name.encode())
                h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.split("(")[0]
    return name.replace("void ", "").strip()


def kernel_stats(path: str) -> dict:
    """{kernel: {calls, total_ns, avg_ns, min_ns, max_ns}} from a rocprofv3 kernel_stats.csv."""
    out = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            n = short_name(row.get("Name", row.get("KernelName", "")))
            out[n] = {"calls": int(row["Calls"]), "total_ns": float(row["TotalDurationNs"]),
                      "avg_ns": float(row["AverageNs"]), "min_ns": float(row["MinNs"]),
                      "max_ns": float(row["MaxNs"])}
    return out


def counter_means(path: str, counter: str) -> dict:
    """{kernel: (dispatches, mean value)} of one counter from a rocprofv3 counter_collection.csv."""
    acc = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            n = short_name(row["Kernel_Name"])
            v = float(row["Counter_Value"])
            c, s = acc.get(n, (0, 0.0))
            acc[n] = (c + 1, s + v)
    return {k: (c, s / c) for k, (c, s) in acc.items()}


def scaled_traffic(fetch_kib: float, write_kib: float, calib: dict) -> float:
    """HBM bytes per dispatch: each counter reading scaled by the copy calibration factor."""
    f = calib["copy_bytes_read"] / (calib["fetch_kib"] * 1024.0)
    w = calib["copy_bytes_written"] / (calib["write_kib"] * 1024.0)
    return fetch_kib * 1024.0 * f + write_kib * 1024.0 * w


def load_traffic(profiles_dir: str, kernel: str, workload: str):
    """Stored HBM traffic per launch for (kernel, workload), or None when absent or when the HIP
    sources changed since the counters were taken."""
    path = os.path.join(profiles_dir, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        db = json.load(fh)
    ent = db.get(f"{kernel}|{workload}")
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent["bytes_per_launch"]


def _main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        st = kernel_stats(argv[1])
        for k, v in sorted(st.items(), key=lambda kv: -kv[1]["total_ns"]):
            print(f"{k:60s} calls={v['calls']:6d} avg={v['avg_ns'] / 1e3:10.2f} us "
                  f"min={v['min_ns'] / 1e3:9.2f} max={v['max_ns'] / 1e3:9.2f}")
    elif len(argv) >= 3 and argv[0] == "counters":
        for k, (n, m) in sorted(counter_means(argv[1], argv[2]).items()):
            print(f"{k:60s} dispatches={n:6d} mean={m:16.1f}")
    elif argv and argv[0] == "hash":
        print(source_hash())
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(_main(sys.argv[1:]))
