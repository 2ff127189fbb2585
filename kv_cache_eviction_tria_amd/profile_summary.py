"""Summaries of rocprofv3 databases for the committed profiles.

  python -m kv_cache_eviction_tria_amd.profile_summary trace DB_DIR  > summary.md
  python -m kv_cache_eviction_tria_amd.profile_summary traffic FETCH_DIR WRITE_DIR \\
         WORKLOAD CAL_BYTES OUT_DIR
  python -m kv_cache_eviction_tria_amd.profile_summary counters PATTERN DIR [DIR ...]

`trace` lists the average duration of every kernel of a --kernel-trace run.
`--skip-first N` (any mode) leaves out each library kernel's first N dispatches,
e.g. the initial pass of the paged workload, whose rounds are what is measured.
`counters` lists, for every kernel whose name contains PATTERN, the mean per
dispatch of every counter the --pmc runs in the DIRs collected.
`traffic` turns two --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch)
into HBM bytes per launch of each eviction-pass kernel, each counter scaled by
what it reads for the calibration kernel (bench.py --calibrate-bytes: a uint8
xor that reads and writes CAL_BYTES), and writes traffic_<stage>_<workload>.txt
(JSON) stamped with a digest of the stage's kernel sources, which bench.py
compares before it reports the figure.
"""
from __future__ import annotations

import glob
import hashlib
import json
import os
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
STAGE_SOURCES = {
    "score": ["tria_score.hip", "tria_prep.hip", "tria_internal.h"],
    "select": ["tria_select.hip", "tria_group.h", "tria_internal.h"],
    "compact": ["tria_compact.hip", "tria_internal.h"],
    "holefill": ["tria_holefill.hip", "tria_internal.h"],
}
STAGE_KERNELS = {"score": "score_", "select": "select_kernel", "compact": "compact_flow_kernel"}
CAL_KERNEL = "BitwiseXorFunctor"


def sources_digest(stage):
    h = hashlib.sha256()
    for f in STAGE_SOURCES[stage]:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _dbs(d):
    return sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))


def short(name):
    n = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return n.split("(")[0]


def _columns(c, table):
    return [r[1] for r in c.execute("pragma table_info(%s)" % table)]


LIBRARY_KERNELS = ("tria::", "calib_")  # the library's kernels, as short() names them


def _library(k):
    return k.startswith(LIBRARY_KERNELS)


def trace(d, skip=0):
    """skip: leave out each kernel's first `skip` dispatches (e.g. a one-off first pass).
    Launches of one kernel with several grid layers (z > 1) are listed apart."""
    rows = {}
    for db in _dbs(d):
        c = sqlite3.connect(db)
        cols = _columns(c, "kernels")
        order = "start" if "start" in cols else "rowid"
        z = "grid_z / max(workgroup_z, 1)" if "grid_z" in cols and "workgroup_z" in cols else "1"
        seen = {}
        for name, dur, gz in c.execute("select name, duration, %s from kernels order by %s" %
                                       (z, order)):
            k = short(name)
            if _library(k) and gz and gz > 1:
                k += " (grid z %d)" % gz
            seen[k] = seen.get(k, 0) + 1
            if _library(k) and seen[k] <= skip:
                continue
            a = rows.setdefault(k, [0, 0.0])
            a[0] += 1
            a[1] += dur
    out = ["| kernel | calls | avg us | total us |", "|---|---|---|---|"]
    other = [0, 0.0]
    for k, (n, tot) in sorted(rows.items(), key=lambda x: -x[1][1]):
        if _library(k):
            out.append("| %s | %d | %.1f | %.1f |" % (k, n, tot / n / 1e3, tot / 1e3))
        else:
            other[0] += n
            other[1] += tot
    out.append("| (input generation, restores and cache flushes: torch and runtime kernels) "
               "| %d | | %.1f |" % (other[0], other[1] / 1e3))
    return "\n".join(out)


def counter_means(d, counter, skip=0):
    """full kernel name -> (mean counter value per dispatch, dispatches), leaving out each
    library kernel's first `skip` dispatches."""
    vals = {}
    for db in _dbs(d):
        c = sqlite3.connect(db)
        cols = _columns(c, "counters_collection")
        order = "dispatch_id" if "dispatch_id" in cols else "rowid"
        for name, v in c.execute(
                "select kernel_name, value from counters_collection where counter_name = ? "
                "order by %s" % order, (counter,)):
            vals.setdefault(name, []).append(float(v))
    acc = {}
    for name, vs in vals.items():
        if "tria::" in name:
            vs = vs[skip:]
        if vs:
            acc[name] = (sum(vs) / len(vs), len(vs))
    return acc


def counters(pattern, dirs):
    acc = {}  # kernel -> counter -> (mean, dispatches)
    for d in dirs:
        for db in _dbs(d):
            c = sqlite3.connect(db)
            for name, cn, v, n in c.execute(
                    "select kernel_name, counter_name, avg(value), count(*) from "
                    "counters_collection group by kernel_name, counter_name"):
                if pattern in name:
                    acc.setdefault(short(name), {})[cn] = (float(v), int(n))
    out = []
    for k, cs in sorted(acc.items()):
        out.append("%s:" % k)
        for cn, (v, n) in sorted(cs.items()):
            out.append("    %-32s %16.1f   (mean of %d dispatches)" % (cn, v, n))
    return "\n".join(out)


def traffic(fetch_dir, write_dir, workload, cal_bytes, out_dir, skip=0):
    fetch = counter_means(fetch_dir, "FETCH_SIZE", skip)
    write = counter_means(write_dir, "WRITE_SIZE", skip)
    cal_f = [v for k, (v, n) in fetch.items() if CAL_KERNEL in k]
    cal_w = [v for k, (v, n) in write.items() if CAL_KERNEL in k]
    if not cal_f or not cal_w:
        names = sorted(set(short(k) for k in list(fetch) + list(write)))
        raise SystemExit("calibration kernel not found in the counter runs; kernels: %s" % names)
    f_scale = cal_bytes / (cal_f[0] * 1024.0)
    w_scale = cal_bytes / (cal_w[0] * 1024.0)
    lines = ["calibration: %s over %d bytes read + written; FETCH_SIZE %.0f KiB -> x%.3f, "
             "WRITE_SIZE %.0f KiB -> x%.3f" % (CAL_KERNEL, cal_bytes, cal_f[0], f_scale, cal_w[0],
                                                w_scale)]
    for stage, pat in STAGE_KERNELS.items():
        fk = [(v, n) for k, (v, n) in fetch.items() if pat in k]
        wk = [(v, n) for k, (v, n) in write.items() if pat in k]
        if not fk or not wk:
            continue
        # several instantiations may match: dispatch-weighted mean per launch
        fv = sum(v * n for v, n in fk) / sum(n for v, n in fk)
        wv = sum(v * n for v, n in wk) / sum(n for v, n in wk)
        rec = {"stage": stage, "workload": workload, "sources_sha256_16": sources_digest(stage),
               "fetch_kib_per_launch": fv, "write_kib_per_launch": wv,
               "fetch_scale": f_scale, "write_scale": w_scale,
               "bytes_per_launch": fv * 1024.0 * f_scale + wv * 1024.0 * w_scale}
        path = os.path.join(out_dir, "traffic_%s_%s.txt" % (stage, workload))
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        lines.append("%s: FETCH %.0f KiB, WRITE %.0f KiB per launch -> %.1f MB HBM traffic" % (
            stage, fv, wv, rec["bytes_per_launch"] / 1e6))
    return "\n".join(lines)


if __name__ == "__main__":
    skip = 0
    if "--skip-first" in sys.argv:
        i = sys.argv.index("--skip-first")
        skip = int(sys.argv[i + 1])
        del sys.argv[i:i + 2]
    if sys.argv[1] == "trace":
        print(trace(sys.argv[2], skip))
    elif sys.argv[1] == "counters":
        print(counters(sys.argv[2], sys.argv[3:]))
    elif sys.argv[1] == "traffic":
        print(traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), sys.argv[6], skip))
    else:
        raise SystemExit(__doc__)
