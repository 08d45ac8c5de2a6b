#!/usr/bin/env python3
"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python bit_expert_ffn_router_amd/profile_summary.py stats  <kernel_stats.csv> <out.txt> "<command>"
    python bit_expert_ffn_router_amd/profile_summary.py traffic <key> <kernel substring> \
        <copy_fetch.csv> <copy_write.csv> <fetch.csv> <write.csv> <out.json> "<command>" [src ...]

stats:   per-kernel calls / average / min / max duration (microseconds) from a
         `rocprofv3 --kernel-trace --stats -f csv` run.
traffic: HBM bytes per launch of one kernel from two `rocprofv3 --pmc` runs
         (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what
         the same counter reads for a plain 1 GiB device copy (`bench.py
         --copy-calibration`): scale = 1 GiB / copy reading.  The record is
         merged into <out.json> under <key>, tagged with a hash of the kernel's
         source files so that a reader can tell when it has gone stale.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def src_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_expert_ffn_router_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stats(path, out, command):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# rocprofv3 kernel-trace statistics", "# command: " + command,
             "# durations in microseconds", "",
             "%-64s %7s %11s %11s %11s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us",
                                              "pct")]
    for r in rows:
        name = r["Name"]
        if len(name) > 64:
            name = name[:61] + "..."
        lines.append("%-64s %7d %11.2f %11.2f %11.2f %7.2f" % (
            name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    open(out, "w").write("\n".join(lines) + "\n")


def _per_kernel(path, sub):
    vals = []
    for r in csv.DictReader(open(path)):
        if sub in r["Kernel_Name"]:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit("no dispatch of %r in %s" % (sub, path))
    return sum(vals) / len(vals), len(vals)


def traffic(key, sub, cf, cw, f, w, out, command, srcs):
    gib_kib = float(1 << 20)
    copy_f, _ = _per_kernel(cf, "copyBuffer")
    copy_w, _ = _per_kernel(cw, "copyBuffer")
    sf, sw = gib_kib / copy_f, gib_kib / copy_w
    kf, nf = _per_kernel(f, sub)
    kw, nw = _per_kernel(w, sub)
    rec = {
        "kernel": sub, "command": command,
        "fetch_kib_raw": kf, "write_kib_raw": kw, "dispatches": [nf, nw],
        "copy_fetch_kib_per_gib": copy_f, "copy_write_kib_per_gib": copy_w,
        "fetch_scale": sf, "write_scale": sw,
        "bytes_per_launch": (kf * sf + kw * sw) * 1024.0,
        "fetch_bytes_per_launch": kf * sf * 1024.0, "write_bytes_per_launch": kw * sw * 1024.0,
        "source_files": srcs, "source_sha": src_sha(srcs),
    }
    db = json.load(open(out)) if os.path.exists(out) else {}
    db[key] = rec
    json.dump(db, open(out, "w"), indent=1, sort_keys=True)
    print(json.dumps(rec))


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 10 and sys.argv[1] == "traffic":
        traffic(*sys.argv[2:10], sys.argv[10:])
    else:
        raise SystemExit(__doc__)
