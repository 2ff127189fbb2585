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
