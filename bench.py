#!/usr/bin/env python3
"""Benchmark of the TQ2_0 ternary decode matvec on one MI355X.

Step = one decode step of the MiniCPM4-8B-shaped linear stack: 32 layers x
(q 4096x4096, k 256x4096, v 256x4096, o 4096x4096, gate 16384x4096,
up 16384x4096, down 4096x16384), i.e. 224 `tq2_gemv` dispatches back to back
on one stream, each with its own fresh fp16 x.  The 224 dispatches are
captured once as a HIP graph and the graph is replayed once per step.  Inputs
(1.955 GB of packed weights, the activations and outputs) are resident in
HBM before the timed region.  Weights are drawn on the GPU from seeded
generators (codes P = 0.3/0.4/0.3, fp16 scales U[0.005, 0.05], x ~ N(0,1))
and packed by `tq2_pack`.

Printed: one JSON line with the whole-step HBM throughput (algorithmic
bytes: 66/256 B per weight + 2 B per x element + 4 B per output), the
roofline of the dominant kernel (the instantiation that runs the gate and up
projections, timed live with HIP events over its back-to-back launches, and
beside it the kernel-trace duration of the committed rocprofv3 record when
that record was taken on the current kernel source), the CPU oracle timed on
the host on a bounded sample (decode layer 0), which also serves as the
parity gate, and the single-call configurations: each timed over rotating
copies of its weights, checked in full against the CPU oracle on the exact
buffers it times, timed on the CPU oracle (1 thread and all host threads),
and set against a read-only stream of the same bytes.

Beside the metric, `step_fused`: the same weights called as a layer shares
its inputs (q, k, v in one fused call on one x; gate and up in one call; o
and down alone: 128 launches), with layer 0 checked bit for bit against
single calls on the same inputs.

  python bench.py [--steps K] [--warmup W] [--no-cpu] [--probes] [--no-configs]
                  [--configs-only] [--no-fused-step] [--probe-sweep]
                  [--config-calls C] [--config-reps R]
  python bench.py --trace-summary <rocprofv3 output dir> --trace-json <bench JSON line file>
                  --trace-command "<the profiled command>"

Trace markers: before each timed section the bench launches an empty kernel
whose workgroup count names the section (`trace_markers` in the JSON), so
one rocprofv3 kernel trace of the bench splits into per-section kernel
durations; `--trace-summary` (CPU only) turns such a trace into
profiles/matvec_bench_sections_kernel_trace.{md,json}, which later runs on
the same kernel source read back as `us_per_launch_trace` / `trace_us`.
`--counter-summary`, `--counter-table` and `--sweep-summary` (CPU only) write
the calibrated HBM traffic, per-section counter tables and the read-probe
sweep under profiles/ from rocprofv3 --pmc runs and a --probe-sweep line.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8.0 TB/s
LAYERS = 32
PROJ = [("q", 4096, 4096), ("k", 256, 4096), ("v", 256, 4096), ("o", 4096, 4096),
        ("gate", 16384, 4096), ("up", 16384, 4096), ("down", 4096, 16384)]
# launches of the dominant kernel: gate and up (16384x4096) both run
# tq2::k_gemv_f16<8, 1, 512, 0, true> (8 rows per wave, one 4096-wide chunk)
DOMINANT = ("gate", "up")
DOMINANT_KERNEL = "tq2::k_gemv_f16<8, 1, 512, 0, true> (gate and up, 16384x4096)"
TRAFFIC_FILE = "gemv_f16_gate_up_16384x4096_traffic.json"
TRACE_FILE = "matvec_bench_sections_kernel_trace.json"
METRIC = "tq2_gemv achieved HBM GB/s and % of MI355X peak; 224-linear decode steps/sec"
STEP_SEEDS = {"weights": "10000 + 7*layer + proj", "x": "20000 + 7*layer + proj"}

# trace-marker ids (workgroups of the empty marker kernel) of the timed sections
MARK_STEP, MARK_DOMINANT, MARK_FUSED, MARK_FLOOR, MARK_SWEEP, MARK_END = 1, 2, 3, 4, 5, 6
MARK_DOMINANT_PROBE = 7
MARK_CONFIG, MARK_CONFIG_PROBE = 100, 200  # + index of the configuration


def algo_bytes(N, K):
    """Algorithmic bytes of one matvec: 2-bit codes + one fp16 scale per 256
    weights, the fp16 x read once, the fp32 y written once."""
    return N * K * 66 // 256 + 2 * K + 4 * N


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ probes

class Probes:
    """The calibration kernels of libtq2probe.so (not part of the ABI)."""

    def __init__(self, torch):
        self.torch = torch
        lib = ctypes.CDLL(os.path.join(ROOT, "ternary_packed_weight_amd", "libtq2probe.so"))
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.tq2probe_empty.argtypes = [P]
        lib.tq2probe_marker.argtypes = [I32, P]
        lib.tq2probe_read.argtypes = [P, I64, P, P]
        lib.tq2probe_read_gridstride.argtypes = [P, I64, P, I32, P]
        lib.tq2probe_blocked_grid.argtypes = [I64, I32]
        lib.tq2probe_blocked_grid.restype = I64
        lib.tq2probe_read_blocked.argtypes = [P, I64, P, I32, I32, I32, P]
        lib.tq2probe_fill.argtypes = [P, I64, ctypes.c_uint32, I32, P]
        for f in ("tq2probe_empty", "tq2probe_marker", "tq2probe_read", "tq2probe_read_gridstride",
                  "tq2probe_read_blocked", "tq2probe_fill"):
            getattr(lib, f).restype = I32
        self.lib = lib
        self.sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")  # >= any grid used

    def _s(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def marker(self, mid):
        assert self.lib.tq2probe_marker(mid, self._s()) == 0

    def empty(self):
        assert self.lib.tq2probe_empty(self._s()) == 0

    def read(self, ptr, nbytes, variant):
        """One read of nbytes at device address ptr: variant ("gs", blocks) for
        the grid-stride kernel or ("blk", loads, mode, nt) for the blocked one."""
        P = ctypes.c_void_p
        if variant[0] == "gs":
            st = self.lib.tq2probe_read_gridstride(P(ptr), nbytes, P(self.sink.data_ptr()), variant[1], self._s())
        elif variant[0] == "ceiling":
            assert self.lib.tq2probe_blocked_grid(nbytes, 1) <= self.sink.numel()
            st = self.lib.tq2probe_read(P(ptr), nbytes, P(self.sink.data_ptr()), self._s())
        else:
            _, loads, mode, nt = variant
            assert self.lib.tq2probe_blocked_grid(nbytes, loads) <= self.sink.numel()
            st = self.lib.tq2probe_read_blocked(P(ptr), nbytes, P(self.sink.data_ptr()), loads, mode, nt,
                                                self._s())
        assert st == 0, st

    def fill(self, ptr, nbytes, value, blocks=2048):
        assert self.lib.tq2probe_fill(ctypes.c_void_p(ptr), nbytes, value, blocks, self._s()) == 0


# the read-only stream set beside every configuration: tq2probe_read, the
# fastest variant of the sweep at 17.3 MB and within 1.5% of the fastest at
# 34.6 MB and 1 GiB (blocked, one 16-byte global load per thread,
# non-temporal)
READ_CEILING = ("ceiling",)


def variant_name(v):
    if v[0] == "ceiling":
        return "tq2probe_read (blocked 1 loads/thread, global, nt)"
    if v[0] == "gs":
        return f"grid-stride {v[1]} WGs x 256, 4 loads/pass, nt"
    _, loads, mode, nt = v
    how = {0: "buffer", 1: "global", 2: "buffer->LDS"}[mode]
    pol = "nt" if (nt or mode == 2) else "default"
    return f"blocked {loads} loads/thread, {how}, {pol}"


# ----------------------------------------------------------------- helpers

def build_stack(tq2, synth, torch):
    """Seeded weights of all 224 linears, packed on the GPU by tq2_pack."""
    stack = []
    host_layer0 = []
    for l in range(LAYERS):
        for p, (name, N, K) in enumerate(PROJ):
            q, d, _ = synth.torch_problem(10000 + 7 * l + p, N, K)
            W = d.float().repeat_interleave(256, dim=1) * (q.float() - 1.0)
            codes, scales, bad = tq2.tq2_pack(W)
            del W
            x = synth.torch_activations(20000 + 7 * l + p, K)
            y = torch.empty(N, dtype=torch.float32, device="cuda")
            stack.append(dict(name=name, N=N, K=K, codes=codes, scales=scales, x=x, y=y, bad=bad))
            if l == 0:
                host_layer0.append(dict(name=name, N=N, K=K, q=q.cpu().numpy(),
                                        d=d.cpu().numpy(), x=x.cpu().numpy()))
            del q, d
    torch.cuda.synchronize()
    bad = sum(int(e["bad"].item()) for e in stack)
    if bad:
        raise RuntimeError(f"tq2_pack reported {bad} bad blocks on synthetic weights")
    return stack, host_layer0


def capture(torch, launches):
    """Capture a list of launches into one HIP graph (after an eager warm-up)."""
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        for f in launches:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for f in launches:
            f()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps):
    """Per-replay time in microseconds, HIP events around `reps` replays
    (events and replays on torch's current stream)."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _sha(paths):
    h = hashlib.sha256()
    for f in paths:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_source_sha():
    return _sha([os.path.join("ternary_packed_weight_amd", "csrc", f)
                 for f in ("tq2_kernels.hip", "tq2_internal.h")])


SOURCES = ["include/tq2.h", "ternary_packed_weight_amd/csrc/tq2_kernels.hip",
           "ternary_packed_weight_amd/csrc/tq2_internal.h", "ternary_packed_weight_amd/csrc/tq2_api.cpp",
           "ternary_packed_weight_amd/csrc/tq2_probes.hip", "ternary_packed_weight_amd/tq2.py",
           "ternary_packed_weight_amd/synth.py", "ternary_packed_weight_amd/build.py",
           "oracle/tq2_oracle.c", "oracle/__init__.py", "bench.py"]


def provenance(torch):
    """What produced the numbers: source and binary fingerprints, tool and
    runtime versions, the device, the host and the seeds."""
    import subprocess
    rec = {"source_sha": _sha(SOURCES), "kernel_source_sha": kernel_source_sha(),
           "libtq2_sha": _sha(["ternary_packed_weight_amd/libtq2.so"]),
           "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        rec["git_commit"] = r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        rec["git_commit"] = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rec["rocm"] = f.read().strip()
    except OSError:
        rec["rocm"] = None
    p = torch.cuda.get_device_properties(0)
    rec["gpu"] = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
                  "hbm_GiB": round(p.total_memory / 2 ** 30, 1)}
    rec["host_cpu"] = host_cpu()
    rec["host_cpus"] = os.cpu_count()
    rec["seeds"] = {"decode_step": STEP_SEEDS,
                    "configs": {label: seed for label, _, _, _, seed in CONFIGS}}
    return rec


def host_cpu():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def _profile_record(name, sha):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    return rec if rec.get("kernel_source_sha") == sha else None


def traffic_from_profiles(sha):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    rec = _profile_record(TRAFFIC_FILE, sha)
    return None if rec is None else rec.get("traffic_bytes_per_launch")


def trace_from_profiles(sha):
    """The committed kernel-trace record (per-section kernel durations), if it
    was taken on the current kernel source; else None."""
    return _profile_record(TRACE_FILE, sha)


def tol_f16(scales_bits, x_f16, N, K):
    """Per-output bound 2e-3 * sum_k |d_b(k) x_k| + 1e-6 of the fp16 path."""
    import numpy as np
    d = np.abs(scales_bits.view(np.float16).astype(np.float64)).reshape(N, K // 256)
    ax = np.abs(x_f16.astype(np.float64)).reshape(K // 256, 256).sum(axis=1)
    return 2e-3 * (d * ax[None, :]).sum(axis=1) + 1e-6


# ------------------------------------------------------------ CPU oracle leg

def cpu_leg(host_layer0, ys_layer0, min_seconds):
    """Time the CPU oracle on decode layer 0 (7 linears) and check the GPU's
    outputs of that layer against it (per-row tolerance
    2e-3 * sum_k |d_b(k) x_k| + 1e-6)."""
    import numpy as np

    import oracle
    from ternary_packed_weight_amd import synth

    packed = []
    for e in host_layer0:
        dd = np.repeat(e["d"].astype(np.float32), 256, axis=1)
        W = (dd * (e["q"].astype(np.float32) - 1.0)).astype(np.float32)
        codes, scales, bad = oracle.pack(W)
        del W, dd
        packed.append((e, codes, scales))
    layer_bytes = sum(algo_bytes(e["N"], e["K"]) for e in host_layer0)
    reps, t0 = 0, time.perf_counter()
    refs = None
    while True:
        out = [oracle.gemv(c, s, e["N"], e["K"], synth.bits(e["x"])) for (e, c, s) in packed]
        refs = refs or out
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    worst = 0.0
    ok = True
    for (e, c, s), yr, yg in zip(packed, refs, ys_layer0):
        tol = tol_f16(s, e["x"], e["N"], e["K"])
        err = np.abs(yg.astype(np.float64) - yr.astype(np.float64))
        worst = max(worst, float((err / tol).max()))
        ok = ok and bool(np.all(err <= tol))
    cores = oracle.threads()
    # the same work on one thread, on a shorter bounded sample
    oracle.set_threads(1)
    reps1, t1 = 0, time.perf_counter()
    while True:
        for (e, c, s) in packed:
            oracle.gemv(c, s, e["N"], e["K"], synth.bits(e["x"]))
        reps1 += 1
        if time.perf_counter() - t1 >= min_seconds / 3:
            break
    dt1 = time.perf_counter() - t1
    oracle.set_threads(cores)
    cpu = {"value": round(layer_bytes * reps / dt / 1e9, 4), "unit": "GB/s",
           "cores": cores, "kind": "oracle", "cpu_model": host_cpu(), "host_cpus": os.cpu_count(),
           "sample": f"decode layer 0 (7 linears, {sum(e['N'] * e['K'] for e in host_layer0)} weights) "
                     f"x {reps} passes in {dt:.1f} s; plain C oracle, fp64 accumulation, OpenMP over rows",
           "value_1_thread": round(layer_bytes * reps1 / dt1 / 1e9, 4),
           "sample_1_thread": f"the same layer x {reps1} passes in {dt1:.1f} s on one thread"}
    nout = sum(e["N"] for e in host_layer0)
    parity = {"passed": ok, "checked": f"all {nout} outputs of decode layer 0 vs the CPU oracle",
              "max_err_over_tol": round(worst, 6)}
    return cpu, parity


def time_cpu(fn, runs=5):
    """Median wall time (us) of fn() over `runs` runs after one warm-up, at
    all the oracle's threads and at one thread."""
    import numpy as np

    import oracle
    cores = oracle.threads()
    out = {}
    for label, th in (("nproc", cores), ("1_thread", 1)):
        oracle.set_threads(th)
        fn()
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            fn()
            ts.append((time.perf_counter() - t0) * 1e6)
        out[label] = float(np.median(ts))
    oracle.set_threads(cores)
    return out, cores


# --------------------------------------------------------- configurations

CONFIGS = [  # (label, N, K, kind, seed): the single-call configurations, timed with cache rotation
    ("c0 q/k-like 256x4096 fp16", 256, 4096, "f16", 1000),
    ("c1 q/o 4096x4096 fp16", 4096, 4096, "f16", 1001),
    ("c1-out 4096x4096 fp16, x with 0.1% outliers x50", 4096, 4096, "f16_out", 1002),
    ("c2 fused gate+up 2x16384x4096 fp16", 16384, 4096, "gate_up", 1003),
    ("c3 down 4096x16384 int8 (fused quantize)", 4096, 16384, "i8", 1004),
    ("c3q down 4096x16384 int8, pre-quantized x_q (tq2_gemv_i8q)", 4096, 16384, "i8q", 1004),
    ("batched gate 16384x4096, 16 tokens per call (tq2_gemm)", 16384, 4096, "gemm16", 1005),
    ("batched gate 16384x4096, 1 token per call (tq2_gemm)", 16384, 4096, "gemm1", 1005),
    ("batched q/o 4096x4096, 4 tokens per call (tq2_gemm)", 4096, 4096, "gemm4", 1006),
    ("batched q/o 4096x4096, 16 tokens per call (tq2_gemm)", 4096, 4096, "gemm16", 1007),
    ("batched down 4096x16384 int8, 16 tokens per call (tq2_gemm_i8q)", 4096, 16384, "gemm_i8q16", 1008),
    ("batched gate 16384x4096 int8, 16 tokens per call (tq2_gemm_i8q)", 16384, 4096, "gemm_i8q16", 1009),
    ("batched down 4096x16384 int8, 2 tokens per call (tq2_gemm_i8q)", 4096, 16384, "gemm_i8q2", 1010),
    # the adjacent entry points, each a single call on its own shape
    ("next: fused q/k/v 4096+256+256 x 4096 fp16 (tq2_gemv_fused)", 4096, 4096, "qkv", 1006),
    ("next: fused q/k/v 4096+256+256 x 4096 int8 (tq2_gemv_i8_fused)", 4096, 4096, "qkv_i8", 1006),
    ("next: gate+up 2x16384x4096 with SiLU*mul epilogue (tq2_gemv_gate_up_silu)", 16384, 4096, "silu", 1003),
    ("next: down 4096x16384 int8 with int8 output (tq2_gemv_i8_requant)", 4096, 16384, "requant", 1004),
]
QKV_ROWS = (4096, 256, 256)
ROTATION_BYTES = 1.1e9  # > the 256 MB Infinity Cache: every timed call streams from HBM
# Untimed replays before each configuration's timed ones: at least
# WARM_REPLAYS and at least WARM_SECONDS of them.  Each configuration is
# timed right after its CPU parity check and CPU timing, seconds in which the
# GPU idles; its clocks then take longer than a few milliseconds of work to
# come back (measured on MI355X: the fused gate+up timed 9.1-9.3 us in the
# first round after such a pause and 8.3-8.4 us in the rounds after it, with
# 10 warm replays, ~3 ms, before each).
WARM_REPLAYS = 10
WARM_SECONDS = 0.25
REQUANT_S_OUT = 0.05
CPU_TIMED_KINDS = ("f16", "f16_out", "gate_up", "i8", "i8q")
GEMM_TOKENS = {"gemm16": 16, "gemm1": 1, "gemm4": 4}
GEMM_I8_TOKENS = {"gemm_i8q16": 16, "gemm_i8q2": 2}  # tq2_gemm_i8q: pre-quantized int8 tokens


def config_bytes(kind, N, K, rows):
    """Algorithmic bytes of one call of a configuration."""
    if kind == "silu":
        return 2 * N * K * 66 // 256 + 2 * K + 4 * N  # h = silu(gate) * up written once
    if kind == "requant":
        return N * K * 66 // 256 + 2 * K + N  # int8 output
    if kind in GEMM_TOKENS:
        return N * K * 66 // 256 + GEMM_TOKENS[kind] * (2 * K + 4 * N)  # weights once, M x and M y
    if kind in GEMM_I8_TOKENS:
        return N * K * 66 // 256 + GEMM_I8_TOKENS[kind] * (K + 4 * N)  # weights once, M x_q and M y
    if kind == "i8q":
        return N * K * 66 // 256 + 4 * N + K  # x_q read once (1 byte per element)
    return sum(Ni * K * 66 // 256 + 4 * Ni for Ni in rows) + 2 * K  # x read once


class ConfigCase:
    """One configuration: its weights drawn on the GPU (torch's seeded
    generator), packed by tq2_pack, and host copies of the same draws packed
    by the CPU oracle for the parity check."""

    def __init__(self, torch, tq2, synth, label, N, K, kind, seed, want_host):
        import numpy as np
        self.label, self.N, self.K, self.kind, self.seed = label, N, K, kind, seed
        self.rows = QKV_ROWS if kind in ("qkv", "qkv_i8") else ((N, N) if kind in ("gate_up", "silu") else (N,))
        self.mats, self.host = [], []
        x = None
        for i, Ni in enumerate(self.rows):
            q, d, xi = synth.torch_problem(seed + 100 * i, Ni, K)
            W = d.float().repeat_interleave(256, dim=1) * (q.float() - 1.0)
            c, s, bad = tq2.tq2_pack(W)
            del W
            assert int(bad.item()) == 0
            self.mats.append((c, s))
            if want_host:
                self.host.append((q.cpu().numpy(), d.cpu().numpy()))
            x = xi if x is None else x
            del q, d
        if kind == "f16_out":
            x = synth.torch_add_outliers(seed + 50, x)
        self.x = x
        self.x_host = x.cpu().numpy()
        # s = fp32(max|x|) / 100 in fp32 (IEEE division), as the workload states
        self.s = float(np.float32(np.abs(self.x_host.astype(np.float32)).max()) / np.float32(100))
        self.X16 = None
        if kind in GEMM_TOKENS:
            self.X16 = torch.stack([synth.torch_activations(seed + 1 + m, K) for m in range(GEMM_TOKENS[kind])])
        self.XQ = None
        if kind in GEMM_I8_TOKENS:
            # M tokens quantized with one static scale: fp32(max|X|) / 100 over all of them
            self.X16 = torch.stack([synth.torch_activations(seed + 1 + m, K)
                                    for m in range(GEMM_I8_TOKENS[kind])])
            self.s = float(np.float32(np.abs(self.X16.cpu().numpy().astype(np.float32)).max()) / np.float32(100))
            self.XQ = tq2.tq2_quantize_i8(self.X16, self.s)  # all tokens in one call: [M][K]
        self.xq = tq2.tq2_quantize_i8(x, self.s) if kind == "i8q" else None
        self.nbytes = config_bytes(kind, N, K, self.rows)
        self.wbytes = sum(self.rows) * K * 66 // 256

    def out_buffer(self, torch):
        if self.kind in GEMM_TOKENS:
            return torch.empty(GEMM_TOKENS[self.kind], self.N, dtype=torch.float32, device="cuda")
        if self.kind in GEMM_I8_TOKENS:
            return torch.empty(GEMM_I8_TOKENS[self.kind], self.N, dtype=torch.float32, device="cuda")
        if self.kind == "requant":
            return torch.empty(self.N, dtype=torch.int8, device="cuda")
        if self.kind == "silu":
            return torch.empty(self.N, dtype=torch.float32, device="cuda")
        return torch.empty(sum(self.rows), dtype=torch.float32, device="cuda")

    def call(self, tq2, mats, x, y, ws=None):
        k, N = self.kind, self.N
        if k in ("f16", "f16_out"):
            return tq2.tq2_gemv(mats[0][0], mats[0][1], x, y=y)
        if k == "gate_up":
            return tq2.tq2_gemv_gate_up(mats[0][0], mats[0][1], mats[1][0], mats[1][1], x, y=y)
        if k in GEMM_TOKENS:
            return tq2.tq2_gemm(mats[0][0], mats[0][1], x, y=y, ws=ws)
        if k in GEMM_I8_TOKENS:
            return tq2.tq2_gemm_i8q(mats[0][0], mats[0][1], x, self.s, y=y, ws=ws)
        if k == "qkv":
            return tq2.tq2_gemv_fused(mats, x, y=y)
        if k == "qkv_i8":
            return tq2.tq2_gemv_i8_fused(mats, x, self.s, y=y)
        if k == "silu":
            return tq2.tq2_gemv_gate_up_silu(mats[0][0], mats[0][1], mats[1][0], mats[1][1], x, h=y)
        if k == "requant":
            return tq2.tq2_gemv_i8_requant(mats[0][0], mats[0][1], x, self.s, REQUANT_S_OUT, y_q=y,
                                           want_deq=False)
        if k == "i8q":
            return tq2.tq2_gemv_i8q(mats[0][0], mats[0][1], x, self.s, y=y)
        assert k == "i8"
        return tq2.tq2_gemv_i8(mats[0][0], mats[0][1], x, self.s, y=y)

    def activation(self):
        if self.kind in GEMM_TOKENS:
            return self.X16
        if self.kind in GEMM_I8_TOKENS:
            return self.XQ
        if self.kind == "i8q":
            return self.xq
        return self.x

    def oracle_parity(self, y_gpu):
        """Every output of one call on the timed buffers (copy 0) against the
        CPU oracle; the oracle packs the host copies of the same draws, and
        its packing must equal tq2_pack's bit for bit.  Returns the record and
        the oracle callables for the CPU timing."""
        import numpy as np

        import oracle
        from ternary_packed_weight_amd import synth
        K = self.K
        packed = []
        for (q, d), (c, s) in zip(self.host, self.mats):
            dd = np.repeat(d.astype(np.float32), 256, axis=1)
            W = (dd * (q.astype(np.float32) - 1.0)).astype(np.float32)
            ch, sh, bad = oracle.pack(W)
            del W, dd
            assert bad == 0
            if not (np.array_equal(ch, c.cpu().numpy()) and np.array_equal(sh, s.cpu().numpy().view(np.uint16))):
                raise RuntimeError(f"{self.label}: tq2_pack differs from the oracle's packing")
            packed.append((ch, sh))
        xb = synth.bits(self.x_host)
        yg = y_gpu.cpu().numpy()
        rec = {"outputs_checked": int(yg.size), "pack_bit_exact": True}
        kind = self.kind
        if kind in ("f16", "f16_out", "gate_up", "qkv"):
            fns, worst, off = [], 0.0, 0
            for (ch, sh), Ni in zip(packed, self.rows):
                ref = oracle.gemv(ch, sh, Ni, K, xb)
                tol = tol_f16(sh, self.x_host, Ni, K)
                err = np.abs(yg.reshape(-1)[off:off + Ni].astype(np.float64) - ref)
                worst = max(worst, float((err / tol).max()))
                fns.append(lambda ch=ch, sh=sh, Ni=Ni: oracle.gemv(ch, sh, Ni, K, xb))
                off += Ni
            rec.update(rule="|y - y_oracle| <= 2e-3 sum_k |d_b(k) x_k| + 1e-6 per output",
                       max_err_over_tol=round(worst, 6), passed=worst <= 1.0)
        elif kind in ("i8", "qkv_i8", "requant"):
            ok, off, fns = True, 0, []
            for (ch, sh), Ni in zip(packed, self.rows):
                ref = oracle.gemv_i8(ch, sh, Ni, K, xb, self.s)
                fns.append(lambda ch=ch, sh=sh, Ni=Ni: oracle.gemv_i8(ch, sh, Ni, K, xb, self.s))
                if kind == "requant":
                    yq_ref, _ = oracle.requant_i8(ref, np.float32(REQUANT_S_OUT))
                    ok = ok and np.array_equal(yg, yq_ref)
                else:
                    ok = ok and np.array_equal(yg[off:off + Ni].view(np.uint32), ref.view(np.uint32))
                off += Ni
            rec.update(rule="bit-exact", passed=bool(ok))
        elif kind == "i8q":
            ch, sh = packed[0]
            xq_ref = oracle.quantize_i8(xb, self.s)
            ok = np.array_equal(self.xq.cpu().numpy(), xq_ref)
            ref, _ = oracle.gemv_i8q(ch, sh, self.N, K, xq_ref, self.s)
            ok = ok and np.array_equal(yg.view(np.uint32), ref.view(np.uint32))
            fns = [lambda: oracle.gemv_i8q(ch, sh, self.N, K, xq_ref, self.s)]
            rec.update(rule="bit-exact (x_q and y)", passed=bool(ok))
        elif kind == "silu":
            (cg, sg), (cu, su) = packed
            g = oracle.gemv(cg, sg, self.N, K, xb).astype(np.float64)
            u = oracle.gemv(cu, su, self.N, K, xb).astype(np.float64)
            tg, tu = tol_f16(sg, self.x_host, self.N, K), tol_f16(su, self.x_host, self.N, K)
            href = oracle.silu_mul(g.astype(np.float32), u.astype(np.float32))
            silu = g / (1 + np.exp(-g))
            bound = 1.1 * tg * (np.abs(u) + tu) + (np.abs(silu) + 1.1 * tg) * tu + 1e-5 * np.abs(href) + 1e-6
            r = float((np.abs(yg.astype(np.float64) - href) / bound).max())
            fns = []
            rec.update(rule="fp16 bounds of g and u propagated through silu(g)*u", max_err_over_bound=round(r, 6),
                       passed=r <= 1.0)
        elif kind in GEMM_I8_TOKENS:
            ch, sh = packed[0]
            Xh = self.X16.cpu().numpy()
            XQ_ref = np.stack([oracle.quantize_i8(synth.bits(Xh[m]), self.s) for m in range(Xh.shape[0])])
            ok = np.array_equal(self.XQ.cpu().numpy(), XQ_ref)
            ref = oracle.gemm_i8q(ch, sh, self.N, K, XQ_ref, self.s)
            ok = ok and np.array_equal(yg.view(np.uint32), ref.view(np.uint32))
            fns = []
            rec.update(rule="bit-exact (x_q of every token and y)", passed=bool(ok))
        else:
            assert kind in GEMM_TOKENS
            ch, sh = packed[0]
            Xh = self.X16.cpu().numpy()
            ref = oracle.gemm(ch, sh, self.N, K, synth.bits(Xh))
            worst = 0.0
            for m in range(GEMM_TOKENS[kind]):
                tol = tol_f16(sh, Xh[m], self.N, K)
                worst = max(worst, float((np.abs(yg[m].astype(np.float64) - ref[m]) / tol).max()))
            fns = []
            rec.update(rule="fp16 bound per token and output", max_err_over_tol=round(worst, 6),
                       passed=worst <= 1.0)
        return rec, fns


def rotation(nbytes, max_calls):
    """(copies, calls per graph): copies of the call's buffers totalling at
    least ROTATION_BYTES, and a graph that touches every copy once (unless
    max_calls caps it, for hardware-counter runs)."""
    import math
    ncopy = max(2, int(math.ceil(ROTATION_BYTES / nbytes)))
    return ncopy, (ncopy if max_calls is None else min(ncopy, max_calls))


def warm(torch, g):
    """Untimed replays of g: at least WARM_REPLAYS, and until at least
    WARM_SECONDS have passed (synchronizing every few replays, so that the
    host clock follows the GPU)."""
    t0 = time.perf_counter()
    n = 0
    while n < WARM_REPLAYS or time.perf_counter() - t0 < WARM_SECONDS:
        g.replay()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_rotating(torch, probes, calls, reps, mark):
    """Median and 95th percentile (us per call) over `reps` replays of one
    graph holding every call once, after the untimed replays of warm()."""
    import numpy as np
    g = capture(torch, calls)
    warm(torch, g)
    if probes is not None:
        probes.marker(mark)
    ts = [time_graph(torch, g, 1) / len(calls) for _ in range(reps)]
    if probes is not None:
        probes.marker(MARK_END)
    del g
    return float(np.median(ts)), float(np.percentile(ts, 95))


def read_ceiling(torch, probes, rb, ncall, reps, variant, mark):
    """us per read of rb bytes from a rotating pool of ncall copies (the
    read-only stream beside a configuration)."""
    pool = torch.ones(ncall * rb, dtype=torch.uint8, device="cuda")
    calls = [lambda j=j: probes.read(pool.data_ptr() + j * rb, rb, variant) for j in range(ncall)]
    us, _ = time_rotating(torch, probes, calls, reps, mark)
    del pool, calls
    torch.cuda.empty_cache()
    return us


def time_configs(torch, tq2, synth, probes, reps, max_calls, with_cpu):
    """Each configuration: parity of one call on the exact buffers timed
    against the CPU oracle (with_cpu), then C rotating copies of the weights
    (>= 1.1 GB in all; x and y rotate with them) captured as one graph that
    calls every copy once, median and p95 over `reps` replays; beside it a
    read-only stream of the call's weight bytes over the same rotation, and
    the CPU oracle's time for the same call (1 thread and all threads)."""
    out = {}
    for ci, (label, N, K, kind, seed) in enumerate(CONFIGS):
        case = ConfigCase(torch, tq2, synth, label, N, K, kind, seed, want_host=with_cpu)
        rec = {"bytes_per_call": int(case.nbytes)}
        ws = None
        if kind in GEMM_I8_TOKENS:
            ws = torch.empty(max(256, tq2.tq2_gemm_i8q_workspace_bytes(N, K, GEMM_I8_TOKENS[kind])),
                             dtype=torch.uint8, device="cuda")
        if kind in GEMM_TOKENS:
            ws = torch.empty(max(256, tq2.tq2_gemm_workspace_bytes(N, K, GEMM_TOKENS[kind])), dtype=torch.uint8,
                             device="cuda")
        # parity and CPU timing on copy 0 (the originally packed buffers)
        if with_cpu:
            y0 = case.out_buffer(torch)
            case.call(tq2, case.mats, case.activation(), y0, ws)
            torch.cuda.synchronize()
            rec["parity"], fns = case.oracle_parity(y0)
            if not rec["parity"]["passed"]:
                raise RuntimeError(f"{label}: parity failed {rec['parity']}")
            if kind in CPU_TIMED_KINDS:
                t, cores = time_cpu(lambda: [f() for f in fns])
                rec["cpu_oracle"] = {"us_per_call_nproc": round(t["nproc"], 1), "threads": cores,
                                     "us_per_call_1_thread": round(t["1_thread"], 1),
                                     "GB_s_nproc": round(case.nbytes / t["nproc"] / 1e3, 4),
                                     "GB_s_1_thread": round(case.nbytes / t["1_thread"] / 1e3, 4),
                                     "runs": "median of 5 after 1 warm-up"}
        ncopy, ncall = rotation(case.nbytes, max_calls)
        copies = [[(c.clone(), s.clone()) for (c, s) in case.mats] for _ in range(ncall)]
        acts = [case.activation().clone() for _ in range(ncall)]
        ys = [case.out_buffer(torch) for _ in range(ncall)]
        calls = [lambda j=j: case.call(tq2, copies[j], acts[j], ys[j], ws) for j in range(ncall)]
        us, us95 = time_rotating(torch, probes, calls, reps, MARK_CONFIG + ci)
        del calls, copies, acts, ys
        torch.cuda.empty_cache()
        rb = (case.wbytes + 255) // 256 * 256  # the call's weight bytes
        us_rd = read_ceiling(torch, probes, rb, ncall, reps, READ_CEILING, MARK_CONFIG_PROBE + ci)
        gbs = case.nbytes / us / 1e3
        rec.update({"us_per_call": round(us, 3), "us_per_call_p95": round(us95, 3),
                    "GB_s": round(gbs, 1), "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
                    "read_probe_us": round(us_rd, 3), "read_probe_GB_s": round(rb / us_rd / 1e3, 1),
                    "pct_of_read_probe": round(100 * us_rd / us, 1),
                    "rotation_copies": ncopy, "calls_per_graph": ncall,
                    "bytes_rotated": int(ncall * case.nbytes), "trace_marker": MARK_CONFIG + ci})
        if kind in GEMM_TOKENS or kind in GEMM_I8_TOKENS:
            rec["tokens_per_s"] = round({**GEMM_TOKENS, **GEMM_I8_TOKENS}[kind] * 1e6 / us, 1)
        if "cpu_oracle" in rec:
            rec["gpu_speedup_vs_cpu_nproc"] = round(rec["cpu_oracle"]["us_per_call_nproc"] / us, 1)
        out[label] = rec
        log(f"{label}: {us:.2f} us/call, {gbs:.1f} GB/s ({gbs / PEAK_HBM_GBS:.1%}); read probe {us_rd:.2f} us"
            + (f"; parity {rec['parity']}" if "parity" in rec else ""))
        del case
        torch.cuda.empty_cache()
    return out


def dispatch_floor(torch, probes, n=400, reps=10):
    """us per graph node of an empty kernel, n nodes back to back."""
    import numpy as np
    g = capture(torch, [probes.empty for _ in range(n)])
    time_graph(torch, g, 3)
    probes.marker(MARK_FLOOR)
    us = float(np.median([time_graph(torch, g, 1) / n for _ in range(reps)]))
    probes.marker(MARK_END)
    return us


def probe_sweep(torch, probes, reps=5):
    """The read-only stream at three sizes (the c3/gate weight bytes, the c2
    weight bytes, 1 GiB), each over rotating copies totalling >= 1.1 GB, for
    every probe variant; us per read and GB/s."""
    sizes = [17_301_504, 34_603_008, 1 << 30]
    variants = [("gs", b) for b in (512, 1024, 2048, 4096, 8192)]
    variants += [("blk", u, m, nt) for m in (0, 1) for nt in (1, 0) for u in (1, 2, 4, 8, 16)]
    variants += [("blk", u, 2, 1) for u in (1, 2, 4, 8)]
    rows = []
    probes.marker(MARK_SWEEP)
    for nbytes in sizes:
        ncopy, ncall = rotation(nbytes, None)
        pool = torch.ones(ncopy * nbytes, dtype=torch.uint8, device="cuda")
        for v in variants:
            calls = [lambda j=j, v=v: probes.read(pool.data_ptr() + j * nbytes, nbytes, v) for j in range(ncall)]
            us, _ = time_rotating(torch, None, calls, reps, 0)
            rows.append({"bytes": nbytes, "variant": variant_name(v), "key": list(v), "us": round(us, 3),
                         "GB_s": round(nbytes / us / 1e3, 1)})
            log(f"sweep {nbytes} B {variant_name(v)}: {us:.3f} us, {nbytes / us / 1e3:.1f} GB/s")
        del pool
        torch.cuda.empty_cache()
    probes.marker(MARK_END)
    return rows


# --------------------------------------------------------------- the step

def fused_step(torch, tq2, stack, steps, probes):
    """The same 224 weights as the step, called the way a model's layer
    shares its inputs: q, k and v in one tq2_gemv_fused call on one x, o
    alone, gate and up in one tq2_gemv_gate_up call on one x, down alone
    (4 launches per layer).  Layer 0's outputs must equal single tq2_gemv
    calls on the same inputs bit for bit."""
    layers = [stack[i:i + len(PROJ)] for i in range(0, len(stack), len(PROJ))]
    bufs, launches, nbytes = [], [], 0
    for q, k, v, o, g, u, d in layers:
        yqkv = torch.empty(q["N"] + k["N"] + v["N"], dtype=torch.float32, device="cuda")
        ygu = torch.empty(2, g["N"], dtype=torch.float32, device="cuda")
        mats = [(q["codes"], q["scales"]), (k["codes"], k["scales"]), (v["codes"], v["scales"])]
        launches += [lambda mats=mats, x=q["x"], y=yqkv: tq2.tq2_gemv_fused(mats, x, y=y),
                     lambda e=o: tq2.tq2_gemv(e["codes"], e["scales"], e["x"], y=e["y"]),
                     lambda g=g, u=u, y=ygu: tq2.tq2_gemv_gate_up(g["codes"], g["scales"], u["codes"],
                                                                  u["scales"], g["x"], y=y),
                     lambda e=d: tq2.tq2_gemv(e["codes"], e["scales"], e["x"], y=e["y"])]
        bufs.append((yqkv, ygu))
        w = sum(e["N"] * e["K"] * 66 // 256 for e in (q, k, v, o, g, u, d))
        nbytes += w + 2 * (q["K"] + o["K"] + g["K"] + d["K"]) + 4 * sum(e["N"] for e in (q, k, v, o, g, u, d))
    graph = capture(torch, launches)
    time_graph(torch, graph, 20)  # untimed warm-up replays
    probes.marker(MARK_FUSED)
    us = time_graph(torch, graph, steps)
    probes.marker(MARK_END)
    q, k, v, o, g, u, d = layers[0]
    yqkv, ygu = bufs[0]
    ref = torch.cat([tq2.tq2_gemv(e["codes"], e["scales"], q["x"]) for e in (q, k, v)])
    ref_gu = torch.stack([tq2.tq2_gemv(e["codes"], e["scales"], g["x"]) for e in (g, u)])
    torch.cuda.synchronize()
    same = bool(torch.equal(yqkv, ref) and torch.equal(ygu, ref_gu))
    log(f"fused step: {us:.1f} us ({1e6 / us:.0f} steps/s), {nbytes / us / 1e3:.1f} GB/s; "
        f"layer 0 equal to single calls: {same}")
    if not same:
        raise RuntimeError("fused calls differ from single calls on layer 0")
    return {"us_per_step": round(us, 1), "steps_per_s": round(1e6 / us, 1),
            "GB_s": round(nbytes / us / 1e3, 1), "bytes_per_step": nbytes,
            "launches_per_step": len(launches), "layer0_equals_single_calls": same,
            "calls": "per layer: tq2_gemv_fused(q,k,v; one x), tq2_gemv(o), "
                     "tq2_gemv_gate_up(gate,up; one x), tq2_gemv(down)"}


# ----------------------------------------------------- trace summary (CPU)

def _find_csv(path, suffix):
    """The one <...>suffix (or suffix.gz) file under a directory, or path."""
    if not os.path.isdir(path):
        return path
    cands = [os.path.join(dp, f) for dp, _, fs in os.walk(path) for f in fs
             if f.endswith(suffix) or f.endswith(suffix + ".gz")]
    if len(cands) != 1:
        raise SystemExit(f"expected one *{suffix} under {path}, found {cands}")
    return cands[0]


def _open_csv(path):
    import gzip
    return gzip.open(path, "rt", newline="") if path.endswith(".gz") else open(path, newline="")


def _read_trace_rows(path):
    import csv
    path = _find_csv(path, "kernel_trace.csv")
    with _open_csv(path) as f:
        rows = list(csv.DictReader(f))
    grid_key = next(k for k in ("Grid_Size_X", "Grid_Size", "Grid_Sizes_X") if k in rows[0])
    wg_key = next(k for k in ("Workgroup_Size_X", "Workgroup_Size", "Workgroup_Sizes_X") if k in rows[0])
    out = []
    for r in rows:
        out.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"],
                    int(r[grid_key]), int(r[wg_key])))
    out.sort()
    return out, path


def trace_summary(trace_path, bench_json_path, command):
    """Split a rocprofv3 kernel trace of bench.py at its marker kernels and
    write profiles/matvec_bench_sections_kernel_trace.{md,json}."""
    import numpy as np
    with open(bench_json_path) as f:
        line = next(ln for ln in f if ln.startswith("{"))
    bench = json.loads(line)
    markers = {int(k): v for k, v in bench["trace_markers"].items()}
    rows, csv_path = _read_trace_rows(trace_path)
    sections = {}
    current = None
    for start, end, name, grid, wg in rows:
        if "k_empty" in name and wg == 64 and (grid // 64) in markers:
            current = markers[grid // 64]  # None: the end of a timed section
            continue
        if current is None:
            continue
        sections.setdefault(current, {}).setdefault((name, grid), []).append((end - start) / 1e3)
    rec = {"kernel_source_sha": bench["provenance"]["kernel_source_sha"],
           "source_sha": bench["provenance"]["source_sha"], "command": command,
           "gpu": bench["provenance"]["gpu"], "sections": {}}
    md = ["# Kernel durations per timed section of bench.py (rocprofv3 kernel trace)", "",
          "Command (on the MI355X, from the repository root):", "", "    " + command, "",
          f"Kernel source sha {rec['kernel_source_sha']} (source sha {rec['source_sha']}); "
          f"{bench['provenance']['gpu']['name']} {bench['provenance']['gpu']['arch']}.",
          "Each section starts at the bench's marker kernel for it (an empty kernel whose workgroup count",
          "names the section) and holds the kernels launched until the next marker.  Durations are",
          "end minus start timestamp of each dispatch (kernel only; the gap between dispatches is not in them).",
          "", "| section | kernel | grid (threads) | dispatches | mean us | median us | min us | max us |",
          "|---|---|---|---|---|---|---|---|"]
    for sec, kernels in sections.items():
        rec["sections"][sec] = []
        for (name, grid), ds in sorted(kernels.items(), key=lambda kv: -len(kv[1])):
            a = np.array(ds)
            e = {"kernel": name, "grid_threads": grid, "dispatches": int(a.size),
                 "mean_us": round(float(a.mean()), 3), "median_us": round(float(np.median(a)), 3),
                 "min_us": round(float(a.min()), 3), "max_us": round(float(a.max()), 3)}
            rec["sections"][sec].append(e)
            md.append(f"| {sec} | `{name}` | {grid} | {e['dispatches']} | {e['mean_us']} | {e['median_us']} | "
                      f"{e['min_us']} | {e['max_us']} |")
    with open(os.path.join(ROOT, "profiles", TRACE_FILE), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    with open(os.path.join(ROOT, "profiles", "matvec_bench_sections_kernel_trace.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    log(f"summarized {len(rows)} dispatches of {csv_path} into profiles/{TRACE_FILE} and its .md")


def _read_counter_rows(path, counter):
    """(dispatch order, kernel name, grid threads, workgroup, value) of every
    dispatch in a rocprofv3 --pmc CSV for one counter."""
    import csv
    path = _find_csv(path, "counter_collection.csv")
    out = {}
    with _open_csv(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            grid = int(r.get("Grid_Size") or r.get("Grid_Size_X"))
            wg = int(r.get("Workgroup_Size") or r.get("Workgroup_Size_X"))
            prev = out.get(key)
            val = float(r["Counter_Value"]) + (prev[4] if prev else 0.0)  # summed over dimensions
            out[key] = (key, r["Kernel_Name"], grid, wg, val)
    return [out[k] for k in sorted(out)], path


def counter_summary(fetch_path, write_path, bench_json_path, commands):
    """Calibrated HBM traffic of every timed section from two rocprofv3 --pmc
    runs of bench.py --probes (FETCH_SIZE, then WRITE_SIZE), each scaled by
    what the counter reads for the 1 GiB read-only grid-stride stream and the
    256 MiB fill of the same run.  Writes profiles/TRAFFIC_FILE (the dominant
    kernel) and profiles/matvec_bench_sections_hbm_traffic.md (every section)."""
    with open(bench_json_path) as f:
        line = next(ln for ln in f if ln.startswith("{"))
    bench = json.loads(line)
    markers = {int(k): v for k, v in bench["trace_markers"].items()}
    per = {}
    cal = {}
    for counter, path in (("FETCH_SIZE", fetch_path), ("WRITE_SIZE", write_path)):
        rows, _ = _read_counter_rows(path, counter)
        current = None
        for _, name, grid, wg, val in rows:
            if "k_empty" in name and wg == 64 and (grid // 64) in markers:
                current = markers[grid // 64]
                continue
            if "k_read_gridstride" in name or ("k_read(" in name and "blk" not in name):
                cal.setdefault(counter + " read", []).append(val)
            if "k_fill" in name:
                cal.setdefault(counter + " fill", []).append(val)
            if current is None:
                continue
            per.setdefault((current, name, grid), {}).setdefault(counter, []).append(val)
    read_kib = max(cal["FETCH_SIZE read"])
    fill_kib = max(cal["WRITE_SIZE fill"])
    f_fetch = (1 << 30) / 1024 / read_kib
    f_write = (1 << 28) / 1024 / fill_kib
    sha = bench["provenance"]["kernel_source_sha"]
    md = ["# HBM traffic per timed section of bench.py (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated)", "",
          "Commands (on the MI355X, from the repository root):", ""] + ["    " + c for c in commands] + [
          "", f"Kernel source sha {sha}.  Calibration in the same runs: the 1 GiB read-only grid-stride stream "
          f"reads {read_kib:.1f} KiB of FETCH_SIZE (factor {f_fetch:.5f}); the 256 MiB fill writes "
          f"{fill_kib:.1f} KiB of WRITE_SIZE (factor {f_write:.5f}).  Per dispatch, averaged over the section's "
          "dispatches of its most frequent kernel; algorithmic bytes as in the bench line (66/256 B per weight, "
          "x read once, y written once).", "",
          "| section | kernel | dispatches | FETCH KiB | WRITE KiB | calibrated bytes | algorithmic bytes | ratio |",
          "|---|---|---|---|---|---|---|---|"]
    algo = {"dominant kernel": algo_bytes(16384, 4096)}
    for label, rec in (bench.get("configs") or {}).items():
        algo[label] = rec["bytes_per_call"]
    dominant = None
    for (sec, name, grid), d in sorted(per.items(), key=lambda kv: -len(kv[1].get("FETCH_SIZE", []))):
        if sec not in algo or "FETCH_SIZE" not in d or "WRITE_SIZE" not in d:
            continue
        fk = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"])
        wk = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"])
        b = fk * 1024 * f_fetch + wk * 1024 * f_write
        md.append(f"| {sec} | `{_kernel_short(name)}` | {len(d['FETCH_SIZE'])} | {fk:.1f} | {wk:.1f} | {b:,.0f} | "
                  f"{algo[sec]:,} | {b / algo[sec]:.3f} |")
        algo.pop(sec)
        if sec == "dominant kernel":
            dominant = {"kernel": name, "kernel_source_sha": sha, "commands": commands,
                        "fetch_size_kib_per_dispatch": round(fk, 1), "write_size_kib_per_dispatch": round(wk, 1),
                        "dispatches_averaged": len(d["FETCH_SIZE"]),
                        "calibration": {"read_probe": {"kernel": "k_read_gridstride (16-byte non-temporal stream)",
                                                       "bytes": 1 << 30, "fetch_size_kib": round(read_kib, 1),
                                                       "factor": round(f_fetch, 5)},
                                        "fill_probe": {"kernel": "k_fill (16-byte stores)", "bytes": 1 << 28,
                                                       "write_size_kib": round(fill_kib, 1),
                                                       "factor": round(f_write, 5)}},
                        "traffic_bytes_per_launch": int(round(b)),
                        "algorithmic_bytes_per_launch": algo_bytes(16384, 4096),
                        "traffic_over_algorithmic": round(b / algo_bytes(16384, 4096), 4)}
    if dominant is None:
        raise SystemExit("no counters for the dominant-kernel section")
    with open(os.path.join(ROOT, "profiles", TRAFFIC_FILE), "w") as f:
        json.dump(dominant, f, indent=1)
        f.write("\n")
    with open(os.path.join(ROOT, "profiles", "matvec_bench_sections_hbm_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    log(f"traffic of the dominant kernel: {dominant['traffic_over_algorithmic']} x algorithmic")


def _kernel_short(name):
    """A kernel's name without its parameter list."""
    if not name.endswith(")"):
        return name
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        depth += {")": 1, "(": -1}.get(name[i], 0)
        if depth == 0:
            return name[:i]
    return name


def sweep_summary(bench_json_path, command):
    """profiles/read_probe_sweep_17MB_35MB_1GiB.md from a bench run with --probe-sweep."""
    with open(bench_json_path) as f:
        line = next(ln for ln in f if ln.startswith("{"))
    bench = json.loads(line)
    rows = bench["read_probe_sweep"]
    sizes = sorted({r["bytes"] for r in rows})
    variants = []
    for r in rows:
        if r["variant"] not in variants:
            variants.append(r["variant"])
    by = {(r["variant"], r["bytes"]): r for r in rows}
    md = ["# Read-only stream probes (achievable HBM read rate per dispatch)", "",
          "Command (on the MI355X, from the repository root):", "", "    " + command, "",
          f"{bench['provenance']['gpu']['name'] or 'MI355X'} {bench['provenance']['gpu']['arch']}; probe source in "
          f"ternary_packed_weight_amd/csrc/tq2_probes.hip (source sha {bench['provenance']['source_sha']}).  Each "
          "size is read from rotating copies totalling >= 1.1 GB (one graph touches every copy once), median of 5 "
          "replays, us per dispatch with the dispatch included.  An empty kernel costs "
          f"{bench['dispatch_floor_us']} us per graph node in the same run.", "",
          "| variant | " + " | ".join(f"{b / 1e6:.1f} MB us | GB/s | % of 8 TB/s" for b in sizes) + " |",
          "|---|" + "---|---|---|" * len(sizes)]
    for v in variants:
        cells = []
        for b in sizes:
            r = by.get((v, b))
            cells += ([f"{r['us']}", f"{r['GB_s']}", f"{100 * r['GB_s'] / PEAK_HBM_GBS:.1f}"] if r else ["", "", ""])
        md.append(f"| {v} | " + " | ".join(cells) + " |")
    best = {b: min((r for r in rows if r["bytes"] == b), key=lambda r: r["us"]) for b in sizes}
    md += ["", "Fastest per size: " + "; ".join(f"{b / 1e6:.1f} MB: {best[b]['variant']}, {best[b]['us']} us "
                                                 f"({best[b]['GB_s']} GB/s)" for b in sizes) + "."]
    with open(os.path.join(ROOT, "profiles", "read_probe_sweep_17MB_35MB_1GiB.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def counter_table(path, bench_json_path, command, out_name):
    """Mean value of every counter of a rocprofv3 --pmc run of this bench,
    per timed section and kernel (split at the trace markers), as
    profiles/<out_name>."""
    import csv
    with open(bench_json_path) as f:
        line = next(ln for ln in f if ln.startswith("{"))
    bench = json.loads(line)
    markers = {int(k): v for k, v in bench["trace_markers"].items()}
    path = _find_csv(path, "counter_collection.csv")
    rows = {}
    with _open_csv(path) as f:
        for r in csv.DictReader(f):
            key = int(r["Dispatch_Id"])
            e = rows.setdefault(key, {"name": r["Kernel_Name"], "grid": int(r.get("Grid_Size") or r.get("Grid_Size_X")),
                                      "wg": int(r.get("Workgroup_Size") or r.get("Workgroup_Size_X")), "c": {}})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg, names, current = {}, [], None
    for key in sorted(rows):
        e = rows[key]
        if "k_empty" in e["name"] and e["wg"] == 64 and (e["grid"] // 64) in markers:
            current = markers[e["grid"] // 64]
            continue
        if current is None:
            continue
        a = agg.setdefault((current, _kernel_short(e["name"]), e["grid"]), {})
        for c, v in e["c"].items():
            a.setdefault(c, []).append(v)
            if c not in names:
                names.append(c)
    md = [f"# rocprofv3 counters per timed section of bench.py ({', '.join(names)})", "",
          "Command (on the MI355X, from the repository root):", "", "    " + command, "",
          f"Kernel source sha {bench['provenance']['kernel_source_sha']}.  Mean per dispatch over the section's "
          "dispatches, per kernel and grid.", "",
          "| section | kernel | grid (threads) | dispatches | " + " | ".join(names) + " |",
          "|---|---|---|---|" + "---|" * len(names)]
    for (sec, name, grid), a in agg.items():
        n = len(next(iter(a.values())))
        md.append(f"| {sec} | `{name}` | {grid} | {n} | " +
                  " | ".join(f"{sum(a[c]) / len(a[c]):.2f}" if c in a else "" for c in names) + " |")
    with open(os.path.join(ROOT, "profiles", out_name), "w") as f:
        f.write("\n".join(md) + "\n")


def trace_kernel_us(trace, section):
    """Mean kernel duration (us) of the section's most frequent kernel."""
    if not trace or section not in trace["sections"] or not trace["sections"][section]:
        return None, None
    e = trace["sections"][section][0]
    return e["mean_us"], e["kernel"]


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle (its parity gates and timings)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--probes", action="store_true", help="also run the byte-counter calibration kernels")
    ap.add_argument("--no-configs", action="store_true", help="skip the single-call configurations")
    ap.add_argument("--configs-only", action="store_true", help="only the single-call configurations")
    ap.add_argument("--probe-sweep", action="store_true", help="sweep the read-only stream variants")
    ap.add_argument("--config-calls", type=int, default=None,
                    help="cap the calls per configuration graph (hardware-counter runs)")
    ap.add_argument("--config-reps", type=int, default=10, help="timed replays per configuration")
    ap.add_argument("--no-fused-step", action="store_true", help="skip the step built from the fused calls")
    ap.add_argument("--trace-summary", help="(CPU) summarize a rocprofv3 kernel trace of this bench")
    ap.add_argument("--trace-json", help="the bench JSON line of the traced run (with --trace-summary)")
    ap.add_argument("--trace-command", default="", help="the traced command, recorded in the summary")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="(CPU) calibrated HBM traffic from two rocprofv3 --pmc runs of this bench with --probes")
    ap.add_argument("--counter-commands", nargs="*", default=[], help="the two profiled commands")
    ap.add_argument("--sweep-summary", help="(CPU) the read-probe sweep table under profiles/ from a --probe-sweep JSON line")
    ap.add_argument("--counter-table", nargs=2, metavar=("PMC_DIR", "OUT_MD"),
                    help="(CPU) per-section mean of every counter of one rocprofv3 --pmc run")
    args = ap.parse_args()

    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_json, args.trace_command)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary[0], args.counter_summary[1], args.trace_json, args.counter_commands)
        return
    if args.sweep_summary:
        sweep_summary(args.sweep_summary, args.trace_command)
        return
    if args.counter_table:
        counter_table(args.counter_table[0], args.trace_json, args.trace_command, args.counter_table[1])
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from ternary_packed_weight_amd import synth
    from ternary_packed_weight_amd import tq2

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    log(f"device: {torch.cuda.get_device_name(0)}")
    probes = Probes(torch)
    prov = provenance(torch)
    sha = prov["kernel_source_sha"]
    trace = trace_from_profiles(sha)
    floor_us = dispatch_floor(torch, probes)
    log(f"dispatch floor: {floor_us:.3f} us per empty graph node")

    out = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f16", "accumulate": "f32", "data": "synthetic"}
    markers = {MARK_STEP: "decode step", MARK_DOMINANT: "dominant kernel",
               MARK_DOMINANT_PROBE: "read probe: dominant kernel", MARK_FUSED: "step_fused",
               MARK_FLOOR: "dispatch floor", MARK_SWEEP: "read probe sweep", MARK_END: None}
    for ci, c in enumerate(CONFIGS):
        markers[MARK_CONFIG + ci] = c[0]
        markers[MARK_CONFIG_PROBE + ci] = "read probe: " + c[0]

    stack = host_layer0 = None
    if not args.configs_only:
        log("building the 224-linear stack")
        t0 = time.time()
        stack, host_layer0 = build_stack(tq2, synth, torch)
        log(f"stack built and packed on the GPU in {time.time() - t0:.1f} s")

        # ---- the step: 224 dispatches on one stream, as one graph
        def launch(e):
            return lambda: tq2.tq2_gemv(e["codes"], e["scales"], e["x"], y=e["y"])

        step_graph = capture(torch, [launch(e) for e in stack])
        for _ in range(args.warmup):
            step_graph.replay()
        torch.cuda.synchronize()                       # barrier (one rank) + sync
        probes.marker(MARK_STEP)
        t_start = time.perf_counter()
        us_step = time_graph(torch, step_graph, args.steps)
        probes.marker(MARK_END)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        step_bytes = sum(algo_bytes(e["N"], e["K"]) for e in stack)
        gbs = step_bytes / us_step / 1e3
        log(f"step: {us_step:.1f} us ({1e6 / us_step:.0f} steps/s), {gbs:.1f} GB/s; wall {wall:.3f} s")

        # ---- dominant kernel: the gate and up launches back to back
        dom = [e for e in stack if e["name"] in DOMINANT]
        dom_graph = capture(torch, [launch(e) for e in dom])
        time_graph(torch, dom_graph, 20)  # untimed warm-up replays
        probes.marker(MARK_DOMINANT)
        us_dom = time_graph(torch, dom_graph, max(3, args.steps // 2)) / len(dom)
        probes.marker(MARK_END)
        dom_bytes = sum(algo_bytes(e["N"], e["K"]) for e in dom) / len(dom)
        achieved = dom_bytes / us_dom / 1e3
        us_tr, kname = trace_kernel_us(trace, markers[MARK_DOMINANT])
        # the read-only stream of the same weight bytes per launch, over as
        # many distinct buffers as the launches (the same rotation), timed the
        # same way: the achievable ceiling of one dispatch of this size
        de = dom[0]
        rb = (de["N"] * de["K"] * 66 // 256 + 255) // 256 * 256
        us_rd = read_ceiling(torch, probes, rb, len(dom), 10, READ_CEILING, MARK_DOMINANT_PROBE)
        roofline = {"bound": "hbm", "kernel": DOMINANT_KERNEL,
                    "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_from_profiles(sha),
                    "bytes_per_launch": int(dom_bytes), "us_per_launch": round(us_dom, 3),
                    "launches_timed": len(dom), "kernel_source_sha": sha,
                    "us_per_launch_trace": us_tr,
                    "frac_trace": None if us_tr is None else round(dom_bytes / us_tr / 1e3 / PEAK_HBM_GBS, 4),
                    "read_probe_us": round(us_rd, 3), "frac_of_read_probe": round(us_rd / us_dom, 4),
                    "gates": "frac (HIP events over the 64 gate/up launches of one step replayed back to back: "
                             "the decode stream's view); frac_trace is the committed rocprofv3 kernel trace of "
                             "the same section on this kernel source (kernel begin to end, under the tracer)"}
        log(f"dominant kernel: {us_dom:.2f} us/launch, {achieved:.1f} GB/s ({achieved / PEAK_HBM_GBS:.1%})"
            + (f"; trace {us_tr} us" if us_tr else ""))
        out.update({"value": round(gbs, 1), "ms_per_step": round(us_step / 1e3, 4)})
        out["config"] = {"workload": "MiniCPM4-8B decode step: 224 TQ2_0 linears (32 layers x q,k,v,o "
                                     "4096/256/256/4096x4096, gate,up 16384x4096, down 4096x16384), fresh "
                                     "fp16 x per linear, one stream, one HIP graph per step",
                         "bytes_per_step": step_bytes, "launches_per_step": len(stack),
                         "parallelism": "single GPU"}
        out["steps_per_s"] = round(1e6 / us_step, 1)
        out["pct_of_peak_hbm"] = round(100 * gbs / PEAK_HBM_GBS, 2)
        out["roofline"] = roofline
        out["step_fused"] = None if args.no_fused_step else fused_step(torch, tq2, stack, args.steps, probes)
        if args.probes:
            # eager launches too, so per-dispatch counters see the dominant kernel
            for e in dom:
                launch(e)()
            torch.cuda.synchronize()
            buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            for _ in range(3):
                probes.fill(buf.data_ptr(), (1 << 30) // 4, 7)
                probes.read(buf.data_ptr(), 1 << 30, ("gs", 2048))
            torch.cuda.synchronize()
            torch.cuda.synchronize()
            del buf
        del step_graph, dom_graph
        torch.cuda.empty_cache()

    out["dispatch_floor_us"] = round(floor_us, 3)
    if args.probe_sweep:
        out["read_probe_sweep"] = probe_sweep(torch, probes)

    if not args.no_configs:
        with_cpu = not args.no_cpu
        out["configs"] = time_configs(torch, tq2, synth, probes, args.config_reps, args.config_calls, with_cpu)
        out["configs_timing"] = (f"per configuration: one graph calling every rotating copy once; untimed replays "
                                 f"(at least {WARM_REPLAYS}, and at least {WARM_SECONDS} s), then the median and "
                                 f"95th percentile of {args.config_reps} timed replays (HIP events); the read probe "
                                 f"beside it the same way")
        for label, rec in out["configs"].items():
            ci = next(i for i, c in enumerate(CONFIGS) if c[0] == label)
            t_us, kname = trace_kernel_us(trace, label)
            rec["trace_kernel"] = kname
            rec["trace_us"] = t_us
            rec["trace_pct_of_peak_hbm"] = None if t_us is None else round(
                100 * rec["bytes_per_call"] / t_us / 1e3 / PEAK_HBM_GBS, 2)
            if CONFIGS[ci][3] in GEMM_TOKENS:
                # against that many one-token calls of the same shape: the
                # single-call configuration of that shape, or the gate/up
                # launches of the step for 16384x4096
                m = GEMM_TOKENS[CONFIGS[ci][3]]
                N_, K_ = CONFIGS[ci][1], CONFIGS[ci][2]
                one = next((out["configs"][c[0]]["us_per_call"] for c in CONFIGS
                            if c[3] == "f16" and (c[1], c[2]) == (N_, K_) and c[0] in out["configs"]), None)
                if one is None and (N_, K_) == (16384, 4096) and stack is not None:
                    one = out["roofline"]["us_per_launch"]
                if one is not None:
                    rec[f"speedup_vs_{m}_gemv"] = round(m * one / rec["us_per_call"], 2)
            if CONFIGS[ci][3] in GEMM_I8_TOKENS:
                # against that many tq2_gemv_i8q calls of the same shape, where timed
                m = GEMM_I8_TOKENS[CONFIGS[ci][3]]
                N_, K_ = CONFIGS[ci][1], CONFIGS[ci][2]
                one = next((out["configs"][c[0]]["us_per_call"] for c in CONFIGS
                            if c[3] == "i8q" and (c[1], c[2]) == (N_, K_) and c[0] in out["configs"]), None)
                if one is not None:
                    rec[f"speedup_vs_{m}_gemv_i8q"] = round(m * one / rec["us_per_call"], 2)
        c0, c1 = (out["configs"][CONFIGS[i][0]]["us_per_call"] for i in (0, 1))
        qkv = next(out["configs"][c[0]] for c in CONFIGS if c[3] == "qkv")
        qkv["three_single_calls_us"] = round(c1 + 2 * c0, 3)

    cpu, parity = None, None
    if stack is not None and not args.no_cpu:
        ys0 = [stack[i]["y"].cpu().numpy() for i in range(len(PROJ))]
        cpu, parity = cpu_leg(host_layer0, ys0, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads; parity {parity}")
    out["cpu_baseline"] = cpu
    out["parity"] = parity
    out["provenance"] = prov
    out["trace_markers"] = {str(k): v for k, v in markers.items()}
    print(json.dumps(out), flush=True)
    if parity is not None and not parity["passed"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
