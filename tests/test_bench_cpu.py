"""Host logic of bench.py that needs no GPU: the one-GPU refusal and the
traffic record, which is reported only for the sources it was measured on."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
    assert '"metric"' not in r.stdout


def test_traffic_record_follows_the_sources(tmp_path, monkeypatch):
    b = load_bench()
    sha = b.sources_sha256()
    rec = [{"workload": "w", "kernel": "k", "fetch_bytes": 10.0, "write_bytes": 2.0, "sources_sha256": sha}]
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(f))
    assert b.measured_traffic("w", "k") == 12.0
    assert b.measured_traffic("w", "other") is None
    rec[0]["sources_sha256"] = "0" * 64            # measured on other sources: not reported
    f.write_text(json.dumps(rec))
    assert b.measured_traffic("w", "k") is None
    monkeypatch.setattr(b, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert b.measured_traffic("w", "k") is None


def test_committed_traffic_record_is_well_formed():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        recs = json.load(f)
    for r in recs:
        assert r["fetch_bytes"] > 0 and r["write_bytes"] > 0
        assert len(r["sources_sha256"]) == 64
        assert os.path.exists(os.path.join(ROOT, "profiles", r["summary"]))
