"""bench.py on the host: the one-GPU guard (a request for several GPUs exits
with a message before anything touches a device), and the rule that the
roofline's `traffic` comes from the committed counter summary only while the
kernel sources it was taken on are unchanged."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_traffic_only_while_sources_match(tmp_path, monkeypatch):
    bench = _bench()
    rec = {"source_sha256": bench.kernel_source_sha(),
           "kernels": {"k_x": {"fetch_bytes": 1000, "write_bytes": 24}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k_x") == 1024
    assert bench.measured_traffic("k_other") is None
    rec["source_sha256"] = "0" * 64  # counters of other kernel sources
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic("k_x") is None
    f.write_text("not json")
    assert bench.measured_traffic("k_x") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("k_x") is None


def test_committed_traffic_summary_is_self_consistent():
    """Bytes = raw KiB x 1024 x the copy-kernel scale, per kernel; the gate/up
    kernel moved close to its algorithmic bytes (the 8 routed experts x
    13,369,344 B: the shared expert's gate/up runs in the top-k launch)."""
    bench = _bench()
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert 1.9 < rec["fetch_scale"] < 2.1 and rec["write_scale"] == 1.0
    for name, k in rec["kernels"].items():
        assert abs(k["fetch_bytes"] - k["fetch_kib_raw"] * 1024 * rec["fetch_scale"]) <= 0.01 * k["fetch_bytes"] + 64, name
        assert abs(k["write_bytes"] - k["write_kib_raw"] * 1024 * rec["write_scale"]) <= 0.01 * k["write_bytes"] + 64, name
    g = rec["kernels"][bench.DECODE_GATEUP_KERNEL]
    assert g["algorithmic_bytes"] == 8 * 13369344
    assert 1.0 <= (g["fetch_bytes"] + g["write_bytes"]) / (8 * 13369344) < 1.05
    for name, k in rec["kernels"].items():
        if k.get("algorithmic_bytes"):
            assert 1.0 <= (k["fetch_bytes"] + k["write_bytes"]) / k["algorithmic_bytes"] < 1.1, name
