"""Host-side logic of bench.py (no GPU): the byte accounting behind every
GB/s figure, the workload's shape list, the multi-GPU refusal and the rule
that the committed HBM-traffic record is used only for the kernel source it
was taken on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_configurations():
    # 66/256 B per weight, x read once (2 B per element), y written once (4 B per output)
    assert bench.algo_bytes(256, 4096) == 279_552
    assert bench.algo_bytes(4096, 4096) == 4_349_952
    assert bench.algo_bytes(16384, 4096) == 17_375_232
    assert bench.algo_bytes(4096, 16384) == 17_350_656


def test_decode_step_workload():
    assert bench.LAYERS == 32
    assert [p[0] for p in bench.PROJ] == ["q", "k", "v", "o", "gate", "up", "down"]
    per_layer = sum(bench.algo_bytes(N, K) for _, N, K in bench.PROJ)
    assert bench.LAYERS * per_layer == 1_963_524_096
    assert bench.LAYERS * len(bench.PROJ) == 224
    assert all(K % 256 == 0 for _, _, K in bench.PROJ)


def test_traffic_record_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha": "0123456789abcdef", "traffic_bytes_per_launch": 12345}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / bench.TRAFFIC_FILE).write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("0123456789abcdef") == 12345
    assert bench.traffic_from_profiles("fedcba9876543210") is None
    (tmp_path / "profiles" / bench.TRAFFIC_FILE).unlink()
    assert bench.traffic_from_profiles("0123456789abcdef") is None


def test_committed_traffic_record_is_consistent():
    with open(os.path.join(ROOT, "profiles", bench.TRAFFIC_FILE)) as f:
        rec = json.load(f)
    cal = rec["calibration"]
    fetch = rec["fetch_size_kib_per_dispatch"] * 1024 * cal["read_probe"]["factor"]
    write = rec["write_size_kib_per_dispatch"] * 1024 * cal["fill_probe"]["factor"]
    assert abs(fetch + write - rec["traffic_bytes_per_launch"]) <= 1024
    assert rec["algorithmic_bytes_per_launch"] == bench.algo_bytes(16384, 4096)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr
