"""Host-side checks of bench.py: the one-GPU contract and the committed counter
summaries it reads (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summaries_are_well_formed():
    profiles = os.path.join(ROOT, "profiles")
    found = [f for f in os.listdir(profiles) if f.endswith("_traffic.json")]
    assert found, "no committed counter summary"
    for f in found:
        t = json.load(open(os.path.join(profiles, f)))
        for key in ("kernel", "tag", "workload", "csrc_sha256", "read_bytes", "write_bytes", "fetch_scale",
                    "write_scale"):
            assert key in t, f"{f}: {key}"
        assert f == f"{t['workload']}_traffic.json"
        # bytes = counter KiB x calibration scale x 1024, as the note states
        assert abs(t["read_bytes"] - t["fetch_kib"] * t["fetch_scale"] * 1024) < 1e-6 * t["read_bytes"] + 1
        assert abs(t["write_bytes"] - t["write_kib"] * t["write_scale"] * 1024) < 1e-6 * t["write_bytes"] + 1
        # the kernel-trace summary for the same workload sits beside it
        assert os.path.exists(os.path.join(profiles, f"{t['workload']}_kernels.md"))


def test_traffic_is_withheld_for_another_kernel_or_other_sources(tmp_path, monkeypatch):
    wl = "llama3.1-8b-layer-16k"
    t = json.load(open(os.path.join(ROOT, "profiles", f"{wl}_traffic.json")))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / f"{wl}_traffic.json").write_text(json.dumps(t))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "csrc_sha256", lambda: t["csrc_sha256"])
    assert bench.measured_traffic(wl, t["tag"]) == int(round(t["read_bytes"] + t["write_bytes"]))
    assert bench.measured_traffic(wl, "pv/pv_gemm") is None
    monkeypatch.setattr(bench, "csrc_sha256", lambda: "0" * 64)
    assert bench.measured_traffic(wl, t["tag"]) is None
