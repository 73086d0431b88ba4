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


def test_every_configuration_rotates_past_the_infinity_cache():
    # one graph touches every copy once, and the copies total >= 1.1 GB, so
    # no timed call finds its weights in the 256 MB Infinity Cache
    for label, N, K, kind, seed in bench.CONFIGS:
        rows = bench.QKV_ROWS if kind in ("qkv", "qkv_i8") else ((N, N) if kind in ("gate_up", "silu") else (N,))
        nbytes = bench.config_bytes(kind, N, K, rows)
        ncopy, ncall = bench.rotation(nbytes, None)
        assert ncall == ncopy and ncall * nbytes >= bench.ROTATION_BYTES, label
    assert bench.config_bytes("gate_up", 16384, 4096, (16384, 16384)) == 34_742_272
    assert bench.config_bytes("i8", 4096, 16384, (4096,)) == 17_350_656
    assert bench.config_bytes("f16", 256, 4096, (256,)) == 279_552


def test_trace_summary_splits_sections_at_markers(tmp_path, monkeypatch):
    """A synthetic rocprofv3 kernel trace: dispatches are assigned to the
    section of the last marker kernel before them (by start time), and the
    record carries the kernel source of the traced run."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    hdr = ("Kind,Agent_Id,Queue_Id,Kernel_Name,Start_Timestamp,End_Timestamp,"
           "Workgroup_Size_X,Grid_Size_X\n")
    rows = [("(anonymous namespace)::k_empty()", 100, 101, 64, 64 * bench.MARK_DOMINANT),
            ("tq2::k_gemv_f16<8, 1, 512, 0, true>", 200, 5200, 256, 131072),
            ("tq2::k_gemv_f16<8, 1, 512, 0, true>", 6000, 12000, 256, 131072),
            ("(anonymous namespace)::k_empty()", 12100, 12101, 64, 64 * bench.MARK_END),
            ("tq2::k_gemv_f16<8, 1, 512, 0, true>", 12200, 12300, 256, 131072),   # untimed: ignored
            ("(anonymous namespace)::k_empty()", 13000, 13001, 64, 64 * (bench.MARK_CONFIG + 4)),
            ("tq2::k_gemv_i8<4, true, false, 4, 1024, false>", 14000, 20000, 1024, 262144)]
    csv = tmp_path / "run_kernel_trace.csv"
    csv.write_text(hdr + "".join(f"KERNEL_DISPATCH,1,1,\"{n}\",{s},{e},{w},{g}\n" for n, s, e, w, g in rows))
    line = {"trace_markers": {str(bench.MARK_DOMINANT): "dominant kernel", str(bench.MARK_END): None,
                              str(bench.MARK_CONFIG + 4): bench.CONFIGS[4][0]},
            "provenance": {"kernel_source_sha": "abc", "source_sha": "def",
                           "gpu": {"name": "x", "arch": "gfx950"}}}
    js = tmp_path / "b.json"
    js.write_text("log line\n" + json.dumps(line) + "\n")
    bench.trace_summary(str(tmp_path), str(js), "rocprofv3 ...")
    rec = json.loads((tmp_path / "profiles" / bench.TRACE_FILE).read_text())
    assert rec["kernel_source_sha"] == "abc"
    dom = rec["sections"]["dominant kernel"][0]
    assert dom["dispatches"] == 2 and dom["mean_us"] == 5.5 and dom["grid_threads"] == 131072
    assert bench.trace_kernel_us(rec, bench.CONFIGS[4][0]) == (6.0, rows[6][0])
    assert bench.trace_kernel_us(rec, "decode step") == (None, None)


def test_counter_summary_calibrates_and_attributes(tmp_path, monkeypatch):
    """Synthetic rocprofv3 --pmc CSVs: the dominant kernel's FETCH/WRITE are
    averaged over its section, scaled by the probes' factors (the 1 GiB read
    reading half its bytes gives factor 2), and tied to the kernel source."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    hdr = "Dispatch_Id,Kernel_Name,Grid_Size,Workgroup_Size,Counter_Name,Counter_Value\n"

    def csv(counter, rows):
        d = tmp_path / counter
        d.mkdir()
        (d / "run_counter_collection.csv").write_text(
            hdr + "".join(f"{i},\"{n}\",{g},{w},{counter},{v}\n" for i, (n, g, w, v) in enumerate(rows)))
        return str(d)

    dom = "tq2::k_gemv_f16<8, 1, 512, 0, true>(tq2::MatSet, long)"
    common = [("k_empty()", 64 * bench.MARK_DOMINANT, 64, 0)]
    fetch = csv("FETCH_SIZE", common + [(dom, 131072, 256, 8500.0), (dom, 131072, 256, 8520.0),
                                        ("k_empty()", 64 * bench.MARK_END, 64, 0),
                                        ("(anonymous namespace)::k_read_gridstride(x)", 524288, 256, 524288.0),
                                        ("(anonymous namespace)::k_fill(x)", 524288, 256, 0.0)])
    write = csv("WRITE_SIZE", common + [(dom, 131072, 256, 64.0), (dom, 131072, 256, 64.0),
                                        ("k_empty()", 64 * bench.MARK_END, 64, 0),
                                        ("(anonymous namespace)::k_read_gridstride(x)", 524288, 256, 0.0),
                                        ("(anonymous namespace)::k_fill(x)", 524288, 256, 262144.0)])
    js = tmp_path / "b.json"
    js.write_text(json.dumps({"trace_markers": {str(bench.MARK_DOMINANT): "dominant kernel",
                                                str(bench.MARK_END): None},
                              "provenance": {"kernel_source_sha": "abc"}, "configs": {}}) + "\n")
    bench.counter_summary(fetch, write, str(js), ["cmd1", "cmd2"])
    rec = json.loads((tmp_path / "profiles" / bench.TRAFFIC_FILE).read_text())
    assert rec["kernel_source_sha"] == "abc" and rec["dispatches_averaged"] == 2
    assert rec["calibration"]["read_probe"]["factor"] == 2.0
    assert rec["traffic_bytes_per_launch"] == round(8510.0 * 1024 * 2 + 64 * 1024)
    assert bench.traffic_from_profiles("abc") == rec["traffic_bytes_per_launch"]
