"""Host-side logic of bench.py (no GPU): the one-GPU contract, the algorithmic work each
stage is divided by, the choice of the roofline kernel, and the source-hash gate on the
HBM traffic recorded under profiles/."""
import glob
import json
import os
import subprocess
import sys

import pytest

import bench
from sampled_softmax_cross_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_stage_work_is_the_definition():
    w = synth.workload("stage01")
    T, d, P = w.T, w.d, w.P
    work = bench.stage_work(w, P)
    flops = 2.0 * T * P * d
    for k in ("logits", "dx", "dw"):
        assert work[k] == ("mfma", flops)
    ldz = (P + 7) // 8 * 8
    assert work["ce"] == ("hbm", 2.0 * T * ldz * 2 + T * 12)
    # 40 x 3 dW tiles for 256 CUs: every candidate row goes through the k-split reduction
    assert work["scatter"] == ("hbm", P * d * (4.0 + 2))
    # e4m3: bf16 Z read, e4m3 gradient written
    assert bench.stage_work(w, P, e4m3=True)["ce"] == ("hbm", T * ldz * 3.0 + T * 12)


def test_dw_whole_tile_rows():
    # S2-late: 96 x 3 = 288 tiles for 256 CUs -> 255 whole tiles (85 row blocks), the
    # other 2816 rows k-split; with fewer tiles than CUs every row is split
    w = synth.workload("s2late")
    assert bench.dw_split_rows(w, w.P, 256) == w.P - 85 * 256 == 2816
    s2e = synth.workload("s2early")
    assert bench.dw_split_rows(s2e, s2e.P, 256) == s2e.P
    full = synth.workload("full")
    assert bench.dw_split_rows(full, full.V, 256) == full.V - 170 * 256


def test_roofline_takes_the_slowest_stage(monkeypatch):
    w = synth.workload("stage01")
    work = bench.stage_work(w, w.P)
    stage_ms = {"candidates": 0.036, "logits": 0.238, "ce": 0.110, "dx": 0.232, "dw": 0.2515,
                "scatter": 0.0157}
    monkeypatch.setattr(bench, "source_sha", lambda: "0" * 16)
    r = bench.roofline_of(w, stage_ms, work, "bf16", False)
    assert r["kernel"] == "dw" and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(2.0 * w.T * w.P * w.d / 0.2515e-3 / 1e12, abs=0.01)
    assert r["frac"] == pytest.approx(r["achieved"] / 2500.0, abs=1e-4)
    assert r["traffic"] is None  # counters from other kernel sources are not reported
    # an HBM-bound slowest stage is reported in GB/s against the HBM peak
    r = bench.roofline_of(w, {"ce": 0.2, "logits": 0.1}, work, "bf16", False)
    assert r["kernel"] == "ce" and r["bound"] == "hbm" and r["peak"] == 8000.0


def test_recorded_traffic_follows_the_source_hash(monkeypatch):
    path = os.path.join(ROOT, "profiles", "stage01_traffic.json")
    rec = json.load(open(path))
    s = rec["stages"]["dw"]
    monkeypatch.setattr(bench, "source_sha", lambda: rec["source_sha"])
    assert bench.recorded_traffic("stage01", "dw") == s["fetch_bytes"] + s["write_bytes"]
    assert bench.recorded_traffic("stage01", "no_such_stage") is None
    assert bench.recorded_traffic("no_such_workload", "dw") is None
    monkeypatch.setattr(bench, "source_sha", lambda: "f" * 16)
    assert bench.recorded_traffic("stage01", "dw") is None


def test_committed_traffic_records_match_the_kernel_sources():
    """Every committed counter record was taken from the kernels as they are now."""
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")))
    assert files
    sha = bench.source_sha()
    stale = [os.path.basename(f) for f in files if json.load(open(f))["source_sha"] != sha]
    assert not stale, f"re-take the counter runs of {stale} (kernel sources changed)"
