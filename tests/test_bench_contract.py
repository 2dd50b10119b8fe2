"""Host-side checks of bench.py's contract (no GPU): a multi-GPU request is
refused with a message, and HBM traffic figures are reported only for the
kernel sources they were measured on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_only_for_the_measured_sources(tmp_path, monkeypatch):
    files = bench.KERNEL_SOURCES["gateup_tiled"]
    for f in files:
        p = tmp_path / f
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text("source of " + f)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.source_sha(files)
    rec = {"gateup_tiled/prefill": {"source_sha": sha, "bytes_per_launch": 123}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("gateup_tiled", "prefill") == 123
    assert bench.traffic_from_profiles("gateup_tiled", "skew") is None
    # a changed source makes the recorded figure stale
    (tmp_path / files[0]).write_text("edited")
    assert bench.traffic_from_profiles("gateup_tiled", "prefill") is None


def test_recorded_traffic_names_known_kernels():
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for key, v in rec.items():
        if "/" not in key:
            continue
        kernel, _ = key.split("/", 1)
        assert kernel in bench.KERNEL_SOURCES, key
        assert v["bytes_per_launch"] > 0
