"""CPU checks of the bench's host logic: the counter-traffic lookup (HBM bytes
per launch from the FETCH_SIZE / WRITE_SIZE table, used only while the
kernel's translation unit is unchanged since the counters were taken) and
the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _table(tmp_path, shas, entry):
    t = {"unit_sha256": shas, "fetch_scale": 2.0, "write_scale": 1.0,
         "workloads": {"decode": {"layer": entry}}}
    p = tmp_path / "pmc.json"
    p.write_text(json.dumps(t))
    return str(p)


def test_traffic_scales_the_counters(tmp_path, monkeypatch):
    unit = bench.KERNEL_UNIT["layer"]
    p = _table(tmp_path, {unit: bench.unit_source_sha(unit)},
               {"fetch_kib": 1000.0, "write_kib": 300.0, "dispatches": 5})
    monkeypatch.setattr(bench, "TRAFFIC_FILE", p)
    # (1000 KiB x 2 + 300 KiB x 1) per launch
    assert bench.measured_traffic("decode", "layer") == (1000 * 2 + 300) * 1024
    assert bench.measured_traffic("prefill", "layer") is None       # no counters taken
    assert bench.measured_traffic("decode", "fused") is None        # no entry
    assert bench.measured_traffic("decode", "no_such_kernel") is None


def test_traffic_is_null_once_the_sources_change(tmp_path, monkeypatch):
    unit = bench.KERNEL_UNIT["layer"]
    p = _table(tmp_path, {unit: "0" * 64}, {"fetch_kib": 1.0, "write_kib": 1.0, "dispatches": 1})
    monkeypatch.setattr(bench, "TRAFFIC_FILE", p)
    assert bench.measured_traffic("decode", "layer") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("decode", "layer") is None


def test_unit_hash_ignores_comments_only(tmp_path, monkeypatch):
    """The hash covers code, not comments: the same code with other comments
    hashes the same, a changed statement does not."""
    a = "int f() { return 1; }  // one\n/* block */\n"
    b = "int f() { return 1; }  // other words\n"
    c = "int f() { return 2; }\n"
    assert bench._code_only(a).split() == bench._code_only(b).split()
    assert bench._code_only(a).split() != bench._code_only(c).split()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
