"""Summarise rocprofv3 result databases (rocpd SQLite) for this library's kernels.

    python -m structured_sparse_gemm_nm_amd.rocprof_summary trace  <dir>
    python -m structured_sparse_gemm_nm_amd.rocprof_summary counters <dir>...
    python -m structured_sparse_gemm_nm_amd.rocprof_summary traffic <key> <kernel> \
        <source_hash> <profile.md> <FETCH_SIZE dir> <WRITE_SIZE dir>

`trace`: per-kernel call count and mean duration from a --kernel-trace run.
`counters`: per-kernel mean of every collected counter (one directory per
--pmc pass); with SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE in one pass it
also prints MFMA utilisation, busy / (GRBM_GUI_ACTIVE / XCDs x CUs x 4 SIMDs):
GRBM_GUI_ACTIVE comes summed over the XCDs ($NM_XCDS, default 8), the busy
count over every SIMD ($NM_CUS CUs, default 256).  With FETCH_SIZE / WRITE_SIZE passes that include the plain
256 MiB copy of `bench.py --copy-calibration`, it also prints the HBM bytes
per launch of each kernel scaled by the copy's bytes / counter ratio.  The
calibration dispatch is the largest copy-kernel dispatch of each pass (the
profiled command must copy nothing larger than 256 MiB: bench.py --no-peaks).
"""
from __future__ import annotations

import collections
import glob
import json
import os
import sqlite3
import sys

COPY_BYTES = 64 * 1024 * 1024 * 4


def _dbs(path):
    return sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0] if "(" in name else name


def trace(path):
    rows = collections.defaultdict(list)
    for db in _dbs(path):
        con = sqlite3.connect(db)
        for name, start, end in con.execute("select name, start, end from kernels"):
            rows[name].append((end - start) / 1000.0)
    out = []
    for name, d in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        out.append((short(name), len(d), sum(d) / len(d)))
    return out


def counters(paths):
    """Per-kernel mean of each counter, and each counter's value for the
    largest copy-kernel dispatch (the calibration copy)."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    calib = {}
    for path in paths:
        for db in _dbs(path):
            con = sqlite3.connect(db)
            q = "select dispatch_id, kernel_name, counter_name, value from counters_collection"
            per = collections.defaultdict(float)
            names = {}
            for did, kname, cname, val in con.execute(q):
                per[(did, cname)] += val
                names[did] = kname
            for (did, cname), val in per.items():
                agg[short(names[did])][cname].append(val)
                if "copyBuffer" in names[did]:
                    calib[cname] = max(calib.get(cname, 0.0), val)
    means = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in agg.items()}
    return means, calib


def copy_scale(copy):
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if copy.get(c):
            scale[c] = COPY_BYTES / (copy[c] * 1024.0)
    return scale


def traffic(argv):
    """Record one kernel's copy-scaled HBM bytes per launch in profiles/traffic.json
    (the file bench.py reads, keyed by its workload key and the source hash)."""
    key, kernel, source_hash, profile, fetch_dir, write_dir = argv
    res, copy = counters([fetch_dir, write_dir])
    scale = copy_scale(copy)
    match = [k for k in res if kernel in k]
    if len(match) != 1 or len(scale) != 2:
        print(f"need exactly one kernel matching {kernel!r} (found {match}) and both counters")
        return 1
    d = res[match[0]]
    rd = d["FETCH_SIZE"] * 1024.0 * scale["FETCH_SIZE"]
    wr = d["WRITE_SIZE"] * 1024.0 * scale["WRITE_SIZE"]
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = os.path.join(root, "profiles", "traffic.json")
    table = {}
    if os.path.exists(path):
        with open(path) as f:
            table = json.load(f)
    table[key] = {"source_hash": source_hash, "kernel": match[0],
                  "hbm_bytes_per_launch": round(rd + wr), "read_bytes": round(rd),
                  "write_bytes": round(wr), "profile": profile}
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"{key}: {match[0]} read {rd / 1e6:.2f} MB write {wr / 1e6:.2f} MB")
    return 0


def main(argv):
    if len(argv) < 2 or argv[0] not in ("trace", "counters", "traffic"):
        print(__doc__)
        return 2
    if argv[0] == "traffic":
        return traffic(argv[1:])
    if argv[0] == "trace":
        print(f"{'kernel':70s} {'calls':>6s} {'mean_us':>10s}")
        for name, n, us in trace(argv[1]):
            print(f"{name[:70]:70s} {n:6d} {us:10.3f}")
        return 0
    res, copy = counters(argv[1:])
    scale = copy_scale(copy)
    cus = int(os.environ.get("NM_CUS", "256"))
    xcds = int(os.environ.get("NM_XCDS", "8"))
    for k, d in sorted(res.items()):
        line = ", ".join(f"{c}={v:.1f}" for c, v in sorted(d.items()))
        print(f"{k[:90]}: {line}")
        if d.get("SQ_VALU_MFMA_BUSY_CYCLES") and d.get("GRBM_GUI_ACTIVE"):
            cycles = d["GRBM_GUI_ACTIVE"] / xcds
            util = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * cus * 4)
            print(f"    MFMA utilisation {100 * util:.1f}% (busy SIMD cycles / ({cycles:.0f} active "
                  f"cycles x {cus} CUs x 4 SIMDs))")
        hbm = [d[c] * 1024.0 * scale[c] for c in ("FETCH_SIZE", "WRITE_SIZE") if c in d and c in scale]
        if len(hbm) == 2:
            print(f"    HBM bytes per launch (copy-scaled): read {hbm[0]/1e6:.2f} MB, "
                  f"write {hbm[1]/1e6:.2f} MB, total {sum(hbm)/1e6:.2f} MB")
    if scale:
        print(f"copy calibration ({COPY_BYTES}-byte copy, largest copy dispatch: " +
              ", ".join(f"{c}={copy[c]:.1f} KiB" for c in scale) + "; bytes per counter byte: " +
              ", ".join(f"{c} x{v:.3f}" for c, v in scale.items()) + ")")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
