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


def _case(b, wl):
    """A stand-in for a prepared GPU case: the host inputs bench.py keeps."""
    import numpy as np
    import synth
    c = b.Case()
    c.wl = wl
    if wl.layout == "masked":
        c.a3, c.mm = synth.masked_inputs(wl)
        c.touched = int((c.mm > 0).sum())
    else:
        c.x = synth.activations(wl.iseed, wl.T, wl.H)
        c.ids, c.tw = synth.routing(wl)
        c.touched = int(np.unique(c.ids).size)
    return c


def test_cpu_leg_samples_and_parity(monkeypatch):
    """The CPU leg's sample choice, its scaling, and its parity figures on
    scaled-down workloads, with the oracle's own output standing in for the
    GPU's (exact: parity passes) and a perturbed copy (fails)."""
    import numpy as np
    import synth
    from oracle import moe_oracle as O
    b = load_bench()
    monkeypatch.setattr(b, "CPU_SAMPLE_EXPERTS", 6)
    for idx, kw in ((1, dict(E=24, H=128, I=64, T=40)), (3, dict(E=12, H=128, I=64, max_m=8)),
                    (4, dict(E=24, H=128, I=64, T=32))):
        wl = synth.scaled(synth.WORKLOADS[idx], **kw)
        w = synth.stacked_weights(wl)
        c = _case(b, wl)
        kind, sel, rows = b.cpu_sample(c)
        data = {"wl": wl, "touched": c.touched}
        for k in ("x", "ids", "tw", "a3", "mm"):
            if hasattr(c, k):
                data[k] = getattr(c, k)
        if kind == "tokens":
            assert np.array_equal(sel, rows)
            n_exp = np.unique(c.ids[sel]).size
            # the small TP8-like shape runs the whole call
            assert n_exp <= 6 or sel.size == wl.T
            exact = O.moe_indexed(c.x, c.ids, c.tw, w, E=wl.E, tokens=sel)
        else:
            assert len(sel) <= 6 and all(c.mm[e] > 0 for e in sel)
            full = O.moe_masked(c.a3, c.mm, w)
            exact = full[rows]
        base, par = b.cpu_leg(data, w, kind, sel, exact)
        assert par["pass"] and par["rel_fro"] == 0 and par["max_abs_over_rms"] == 0
        assert base["cores"] == b.cpu_cores() and base["value"] > 0 and base["kind"] == "oracle"
        assert par["bf16_floor"] > 0
        _, bad = b.cpu_leg(data, w, kind, sel, exact * (1 + 2e-2))
        assert not bad["pass"]


def test_token_sample_bounds_experts():
    import numpy as np
    b = load_bench()
    ids = np.array([[0, 1], [2, 3], [1, 4], [5, 6]])
    tok, n = b.token_sample(ids, 5)
    assert tok.tolist() == [0, 1, 2] and n == 5
    tok, n = b.token_sample(ids, 1)           # at least one token
    assert tok.tolist() == [0] and n == 2
