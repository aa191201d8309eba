"""Summaries of rocprofv3 output for the benchmark step.

``python -m sparse_top_kl_amd.profiling stats <kernel_stats.csv>``
    per-kernel launches, total and average duration (from
    ``rocprofv3 --kernel-trace --stats -f csv``).

``python -m sparse_top_kl_amd.profiling traffic --fetch <csv> --write <csv>
      --copy-mib M --kernel NAME --workload W [--json profiles/traffic.json]``
    HBM bytes per launch of kernel NAME from two counter runs of the same
    command (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, KiB per dispatch).
    Each counter is scaled by what it reads for the plain device copy of M MiB
    that ``bench.py --copy-calibration-mib M`` performs before timing (the copy
    reads and writes exactly M MiB). With ``--json`` the figure is stored for
    bench.py, keyed by workload, kernel and the hash of the kernel sources.
"""

from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys


def short_name(kernel: str) -> str:
    m = re.search(r"fkl::(k_\w+)", kernel)
    if m:
        return m.group(1)
    return kernel.split("(")[0][-60:]


def kernel_stats(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({
                "kernel": short_name(r["Name"]),
                "calls": int(r["Calls"]),
                "total_ms": float(r["TotalDurationNs"]) / 1e6,
                "avg_ms": float(r["AverageNs"]) / 1e6,
                "min_ms": float(r["MinNs"]) / 1e6,
                "max_ms": float(r["MaxNs"]) / 1e6,
                "percent": float(r["Percentage"]),
            })
    rows.sort(key=lambda x: -x["total_ms"])
    return rows


def counter_per_dispatch(path: str, counter: str):
    """{kernel short name: [value per dispatch, ...]} for one counter."""
    vals = collections.defaultdict(dict)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            k = short_name(r["Kernel_Name"])
            d = int(r["Dispatch_Id"])
            vals[k][d] = vals[k].get(d, 0.0) + float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in vals.items()}


def copy_kernel(per_kernel: dict, expect_kib: float):
    """The calibration copy: the non-library kernel whose reading is closest to
    the copy size (torch's copy kernel has no fixed name)."""
    best = None
    for k, vs in per_kernel.items():
        if k.startswith("k_"):
            continue
        for v in vs:
            if best is None or abs(v - expect_kib) < abs(best[1] - expect_kib):
                best = (k, v)
    if best is None:
        raise SystemExit("no calibration copy dispatch found in the counter output")
    return best


def source_hash(root: str) -> str:
    sys.path.insert(0, root)
    import bench  # noqa: E402
    return bench.source_hash()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--json")
    a = ap.parse_args(argv)

    if a.cmd == "stats":
        rows = kernel_stats(a.csv)
        print(f"{'kernel':18s} {'calls':>6s} {'total ms':>10s} {'avg ms':>9s} {'min ms':>9s} "
              f"{'max ms':>9s} {'%':>6s}")
        for r in rows:
            print(f"{r['kernel']:18s} {r['calls']:6d} {r['total_ms']:10.3f} {r['avg_ms']:9.4f} "
                  f"{r['min_ms']:9.4f} {r['max_ms']:9.4f} {r['percent']:6.2f}")
        return

    copy_kib = a.copy_mib * 1024.0
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, "WRITE_SIZE")
    ck_f, copy_fetch = copy_kernel(fetch, copy_kib)
    ck_w, copy_write = copy_kernel(write, copy_kib)
    f_factor = copy_fetch / copy_kib   # counter KiB per KiB actually read
    w_factor = copy_write / copy_kib
    if a.kernel not in fetch or a.kernel not in write:
        raise SystemExit(f"kernel {a.kernel} missing from the counter output")
    fk = sum(fetch[a.kernel]) / len(fetch[a.kernel])
    wk = sum(write[a.kernel]) / len(write[a.kernel])
    read_b = fk * 1024.0 / f_factor
    write_b = wk * 1024.0 / w_factor
    print(f"copy calibration ({ck_f}): FETCH_SIZE {copy_fetch:.0f} KiB, WRITE_SIZE "
          f"{copy_write:.0f} KiB for {copy_kib:.0f} KiB copied -> factors {f_factor:.4f} / "
          f"{w_factor:.4f}")
    print(f"{a.kernel}: {len(fetch[a.kernel])} dispatches; FETCH_SIZE {fk:.0f} KiB, WRITE_SIZE "
          f"{wk:.0f} KiB per dispatch -> {read_b / 1e9:.3f} GB read + {write_b / 1e9:.3f} GB "
          f"written = {(read_b + write_b) / 1e9:.3f} GB per launch")
    if a.json:
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        data = {}
        if os.path.exists(a.json):
            with open(a.json) as f:
                data = json.load(f)
        data.setdefault(a.workload, {})[a.kernel] = {
            "bytes_per_launch": read_b + write_b,
            "read_bytes_per_launch": read_b,
            "write_bytes_per_launch": write_b,
            "fetch_kib_per_dispatch": fk,
            "write_kib_per_dispatch": wk,
            "copy_factor_fetch": f_factor,
            "copy_factor_write": w_factor,
            "source_hash": source_hash(root),
        }
        with open(a.json, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
        print(f"stored in {a.json}")


if __name__ == "__main__":
    main()
