"""bench.py pieces that run without a GPU: the one-GPU refusal, the roofline
entry's arithmetic, and the rule that counter traffic is reported only when the
committed counter summary was taken on the current kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from kv_cache_eviction_tria_amd.profile_summary import STAGE_SOURCES, sources_digest  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_roofline_entry():
    alg = 1868489568.0
    e = bench.roofline("compact", 0.66, 2, 2 * alg, "no_such_workload")
    assert e["launches_per_step"] == 2 and e["avg_launch_ms"] == pytest.approx(0.33)
    assert e["alg_bytes_per_launch"] == pytest.approx(alg)
    assert e["achieved"] == pytest.approx(alg / 0.33e-3 / 1e9)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["peak"] == 8000.0
    assert e["traffic"] is None  # no counter summary for that workload
    assert bench.roofline("select", 0.07, 1, None, "no_such_workload")["frac"] is None


def test_traffic_only_from_counters_of_the_current_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"stage": "compact", "workload": "w", "bytes_per_launch": 2.5e9,
           "sources_sha256_16": sources_digest("compact")}
    path = tmp_path / "profiles" / "traffic_compact_w.txt"
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("compact", "w") == 2.5e9
    rec["sources_sha256_16"] = "0" * 16  # counters of other sources
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("compact", "w") is None
    assert bench.measured_traffic("score", "w") is None  # no summary at all


def test_committed_counter_summaries_are_well_formed():
    d = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(d) if f.startswith("traffic_") and f.endswith(".txt")]
    assert names
    for f in names:
        rec = json.load(open(os.path.join(d, f)))
        assert rec["stage"] in STAGE_SOURCES and f == "traffic_%s_%s.txt" % (rec["stage"],
                                                                              rec["workload"])
        assert rec["bytes_per_launch"] > 0 and len(rec["sources_sha256_16"]) == 16


def test_trace_summary_lists_library_kernels_by_grid_layers(tmp_path):
    """The trace table names the library's kernels (tria:: and the calibration
    kernels), lists one-launch multi-layer calls apart, and folds the rest."""
    import sqlite3

    from kv_cache_eviction_tria_amd import profile_summary as ps
    db = sqlite3.connect(str(tmp_path / "k_results.db"))
    db.execute("create table kernels (name text, duration int, start int, grid_z int, "
               "workgroup_z int)")
    rows = [("void tria::prep_kernel(int)", 5000, 1, 1, 1),
            ("void tria::prep_kernel(int)", 7000, 2, 1, 1),
            ("void (anonymous namespace)::calib_partial4_kernel<float>(float const*)", 10000, 3, 1, 1),
            ("void (anonymous namespace)::calib_partial4_kernel<float>(float const*)", 240000, 4, 36, 1),
            ("void at::native::elementwise_kernel<int>(int)", 3000, 5, 1, 1)]
    db.executemany("insert into kernels values (?, ?, ?, ?, ?)", rows)
    db.commit()
    db.close()
    out = ps.trace(str(tmp_path)).splitlines()
    assert "| tria::prep_kernel | 2 | 6.0 | 12.0 |" in out
    assert "| calib_partial4_kernel<float> | 1 | 10.0 | 10.0 |" in out
    assert "| calib_partial4_kernel<float> (grid z 36) | 1 | 240.0 | 240.0 |" in out
    assert out[-1].endswith("| 1 | | 3.0 |")
    skipped = ps.trace(str(tmp_path), skip=1).splitlines()
    assert "| tria::prep_kernel | 1 | 7.0 | 7.0 |" in skipped
