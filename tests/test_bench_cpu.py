"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the
statistics it reports, the roofline object's arithmetic, and the rule that a
stored HBM-traffic figure is reported only while its kernels' sources are the
ones it was measured on."""
import json
import os
import subprocess
import sys

import bench
from paged_kv_cache_66_amd import srchash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def test_summary_statistics():
    s = bench.summary([float(x) for x in range(1, 101)])  # 1 .. 100
    assert s["mean"] == 50.5
    assert s["median"] == 51.0   # upper median of an even count
    assert s["p10"] == 11.0 and s["p90"] == 91.0
    one = bench.summary([2.5])
    assert one == {"mean": 2.5, "median": 2.5, "p10": 2.5, "p90": 2.5}


def test_decode_roofline_arithmetic():
    res = {"fused_ms": {"mean": 2.0, "median": 1.9, "p10": 1.8, "p90": 2.2}, "fused_bytes": 8_000_000_000,
           "workload": "w", "kernel": "k"}
    r = bench.decode_roofline(res, 123)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert r["achieved"] == 4000.0          # 8 GB in 2 ms
    assert r["frac"] == 0.5                 # of 8000 GB/s
    assert r["traffic"] == 123
    assert r["avg_launch_ms"] == 2.0 and r["median_launch_ms"] == 1.9
    assert r["p10_p90_launch_ms"] == [1.8, 2.2]


def _write_traffic(tmp_path, monkeypatch, stamp):
    path = tmp_path / "traffic_w.json"
    path.write_text(json.dumps({"bytes_per_launch": 4321, "kernel_sha256": stamp}))
    monkeypatch.setattr(bench, "traffic_file", lambda workload: str(path))


def test_stored_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    for kind in ("decode", "prefill"):
        _write_traffic(tmp_path, monkeypatch, srchash.kernel_sha256(kind))
        assert bench.stored_traffic("w", kind) == 4321
        _write_traffic(tmp_path, monkeypatch, "0" * 64)
        assert bench.stored_traffic("w", kind) is None
    monkeypatch.setattr(bench, "traffic_file", lambda workload: str(tmp_path / "absent.json"))
    assert bench.stored_traffic("w", "decode") is None


def test_committed_traffic_files_are_well_formed():
    for name, kind in (("8b-decode-bs16", "decode"), ("8b-decode-bs256", "decode"),
                       ("qwen3-0.6b-decode", "decode"), ("long-context-decode", "decode"),
                       ("chunked-prefill", "prefill")):
        with open(bench.traffic_file(name)) as f:
            rec = json.load(f)
        assert rec["bytes_per_launch"] == round(sum(k["fetch_bytes"] + k["write_bytes"]
                                                    for k in rec["per_kernel"].values()))
        assert len(rec["kernel_sha256"]) == 64
        assert all(("decode_" if kind == "decode" else "prefill_") in k for k in rec["per_kernel"])
