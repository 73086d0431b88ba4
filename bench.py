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
projections, 39% of the step, timed live with HIP events over its
back-to-back launches) and the CPU oracle
timed on the host on a bounded sample (decode layer 0), which also serves as
the parity gate: a mismatch prints passed=false and exits non-zero.

Beside it, `step_fused`: the same weights called as a layer shares its
inputs (q, k, v in one fused call on one x; gate and up in one call; o and
down alone: 128 launches), with layer 0 checked bit for bit against single
calls on the same inputs.  It is reported, not the metric: the metric's step
gives every linear its own x.

  python bench.py [--steps K] [--warmup W] [--no-cpu] [--probes] [--no-configs]
                  [--no-fused-step] [--config-calls C] [--config-reps R]

--config-calls and --config-reps shrink the single-call configuration graphs
for hardware-counter runs (every dispatch is then profiled); the figures of a
normal run use the defaults.
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
# tq2::k_gemv_f16<8, 1, 512, 0> (8 rows per wave, one 4096-wide chunk)
DOMINANT = ("gate", "up")
DOMINANT_KERNEL = "tq2::k_gemv_f16<8, 1, 512, 0, true> (gate and up, 16384x4096)"
TRAFFIC_FILE = "gemv_f16_gate_up_16384x4096_traffic.json"
METRIC = "tq2_gemv achieved HBM GB/s and % of MI355X peak; 224-linear decode steps/sec"


def algo_bytes(N, K):
    """Algorithmic bytes of one matvec: 2-bit codes + one fp16 scale per 256
    weights, the fp16 x read once, the fp32 y written once."""
    return N * K * 66 // 256 + 2 * K + 4 * N


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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
    """Per-replay time in microseconds, HIP events around `reps` replays."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("tq2_kernels.hip", "tq2_internal.h"):
        with open(os.path.join(ROOT, "ternary_packed_weight_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(sha):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


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
        d = np.abs(s.view(np.float16).astype(np.float64))
        ax = np.abs(e["x"].astype(np.float64)).reshape(-1, 256).sum(axis=1)
        tol = 2e-3 * (d * ax[None, :]).sum(axis=1) + 1e-6
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
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    cpu = {"value": round(layer_bytes * reps / dt / 1e9, 4), "unit": "GB/s",
           "cores": cores, "kind": "oracle", "cpu_model": model, "host_cpus": os.cpu_count(),
           "sample": f"decode layer 0 (7 linears, {sum(e['N'] * e['K'] for e in host_layer0)} weights) "
                     f"x {reps} passes in {dt:.1f} s; plain C oracle, fp64 accumulation, OpenMP over rows",
           "value_1_thread": round(layer_bytes * reps1 / dt1 / 1e9, 4),
           "sample_1_thread": f"the same layer x {reps1} passes in {dt1:.1f} s on one thread"}
    nout = sum(e["N"] for e in host_layer0)
    parity = {"passed": ok, "checked": f"all {nout} outputs of decode layer 0 vs the CPU oracle",
              "max_err_over_tol": round(worst, 6)}
    return cpu, parity


def run_probes(torch, nbytes=1 << 30):
    """Calibration kernels of known size for hardware byte counters: a
    read-only 16-byte stream over `nbytes` and a fill of nbytes/4."""
    lib = ctypes.CDLL(os.path.join(ROOT, "ternary_packed_weight_amd", "libtq2probe.so"))
    lib.tq2probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p]
    lib.tq2probe_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32,
                                  ctypes.c_void_p]
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        lib.tq2probe_fill(ctypes.c_void_p(buf.data_ptr()), nbytes // 4, 7, 2048, s)
        lib.tq2probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), 2048, s)
    torch.cuda.synchronize()
    return {"read_bytes": nbytes, "fill_bytes": nbytes // 4}


CONFIGS = [  # (label, N, K, kind, seed): the single-call configurations, timed with cache rotation
    ("c0 q/k-like 256x4096 fp16", 256, 4096, "f16", 1000),
    ("c1 q/o 4096x4096 fp16", 4096, 4096, "f16", 1001),
    ("c2 fused gate+up 2x16384x4096 fp16", 16384, 4096, "gate_up", 1003),
    ("c3 down 4096x16384 int8 (fused quantize)", 4096, 16384, "i8", 1004),
    ("c3q down 4096x16384 int8, pre-quantized x_q (tq2_gemv_i8q)", 4096, 16384, "i8q", 1004),
    ("batched gate 16384x4096, 16 tokens per call (tq2_gemm)", 16384, 4096, "gemm16", 1005),
    # the adjacent entry points, each a single call on its own shape
    ("next: fused q/k/v 4096+256+256 x 4096 fp16 (tq2_gemv_fused)", 4096, 4096, "qkv", 1006),
    ("next: fused q/k/v 4096+256+256 x 4096 int8 (tq2_gemv_i8_fused)", 4096, 4096, "qkv_i8", 1006),
    ("next: gate+up 2x16384x4096 with SiLU*mul epilogue (tq2_gemv_gate_up_silu)", 16384, 4096, "silu", 1003),
    ("next: down 4096x16384 int8 with int8 output (tq2_gemv_i8_requant)", 4096, 16384, "requant", 1004),
]
QKV_ROWS = (4096, 256, 256)
ROTATION_BYTES = 1.1e9  # > the 256 MB Infinity Cache: every timed call streams from HBM
WARM_REPLAYS = 5  # untimed graph replays (up to 2000 calls) before each configuration's timed ones


def fused_step(torch, tq2, stack, steps):
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
    us = time_graph(torch, graph, steps)
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


def time_configs(torch, tq2, synth, reps=10, max_calls=400):
    """Per-call time of each single-call configuration: C rotating copies of
    the weights (>= 1.1 GB in all; x and y rotate with them), up to 400
    back-to-back calls captured as
    one graph, median and 95th percentile over `reps` replays after
    WARM_REPLAYS untimed ones.  Beside it, a read-only 16-byte
    stream kernel, one dispatch per call reading the call's weight bytes from
    a rotating pool of the same size: the achievable ceiling at that size,
    dispatch floor included."""
    import numpy as np
    probe = ctypes.CDLL(os.path.join(ROOT, "ternary_packed_weight_amd", "libtq2probe.so"))
    probe.tq2probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_void_p]
    probe.tq2probe_read.restype = ctypes.c_int32
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    out = {}
    for label, N, K, kind, seed in CONFIGS:
        rows = QKV_ROWS if kind in ("qkv", "qkv_i8") else ((N, N) if kind in ("gate_up", "silu") else (N,))
        nmat = len(rows)
        mats = []
        xs = None
        for i, Ni in enumerate(rows):
            q, d, x = synth.torch_problem(seed + 100 * i, Ni, K)
            W = d.float().repeat_interleave(256, dim=1) * (q.float() - 1.0)
            c, s, _ = tq2.tq2_pack(W)
            del W, q, d
            mats.append((c, s))
            xs = x if xs is None else xs
        nbytes = sum(Ni * K * 66 // 256 + 4 * Ni for Ni in rows) + 2 * K  # x read once
        if kind == "silu":
            nbytes = 2 * N * K * 66 // 256 + 2 * K + 4 * N  # h = silu(gate) * up written once
        if kind == "requant":
            nbytes = N * K * 66 // 256 + 2 * K + N  # int8 output
        if kind == "gemm16":
            nbytes = N * K * 66 // 256 + 16 * (2 * K + 4 * N)  # weights once, 16 x and 16 y
        if kind == "i8q":
            nbytes = N * K * 66 // 256 + 4 * N + K  # x_q read once (1 byte per element)
        ncopy = max(2, int(np.ceil(ROTATION_BYTES / nbytes)))
        copies = [[(c.clone(), s.clone()) for (c, s) in mats] for _ in range(ncopy)]
        del mats
        ncall = min(ncopy, max_calls)
        # x and y rotate with the weights (one copy per call in the graph), so
        # every call reads its activations from memory rather than from a
        # cache that the previous call warmed
        ys = [torch.empty(sum(rows), dtype=torch.float32, device="cuda") for _ in range(ncall)]
        xr = [xs.clone() for _ in range(ncall)]
        sc = float(xs.float().abs().max() / 100)
        if kind == "f16":
            calls = [lambda j=j: tq2.tq2_gemv(copies[j][0][0], copies[j][0][1], xr[j], y=ys[j])
                     for j in range(ncall)]
        elif kind == "gate_up":
            calls = [lambda j=j: tq2.tq2_gemv_gate_up(copies[j][0][0], copies[j][0][1], copies[j][1][0],
                                                      copies[j][1][1], xr[j], y=ys[j].view(2, N))
                     for j in range(ncall)]
        elif kind == "gemm16":
            X16 = torch.stack([synth.torch_activations(seed + 1 + m, K) for m in range(16)])
            X16r = [X16.clone() for _ in range(ncall)]
            Y16 = [torch.empty(16, N, dtype=torch.float32, device="cuda") for _ in range(ncall)]
            ws16 = torch.empty(tq2.tq2_gemm_workspace_bytes(N, K, 16), dtype=torch.uint8, device="cuda")
            calls = [lambda j=j: tq2.tq2_gemm(copies[j][0][0], copies[j][0][1], X16r[j], y=Y16[j], ws=ws16)
                     for j in range(ncall)]
        elif kind == "qkv":
            calls = [lambda j=j: tq2.tq2_gemv_fused(copies[j], xr[j], y=ys[j]) for j in range(ncall)]
        elif kind == "qkv_i8":
            calls = [lambda j=j: tq2.tq2_gemv_i8_fused(copies[j], xr[j], sc, y=ys[j]) for j in range(ncall)]
        elif kind == "silu":
            calls = [lambda j=j: tq2.tq2_gemv_gate_up_silu(copies[j][0][0], copies[j][0][1], copies[j][1][0],
                                                           copies[j][1][1], xr[j], h=ys[j][:N])
                     for j in range(ncall)]
        elif kind == "requant":
            yq = [torch.empty(N, dtype=torch.int8, device="cuda") for _ in range(ncall)]
            calls = [lambda j=j: tq2.tq2_gemv_i8_requant(copies[j][0][0], copies[j][0][1], xr[j], sc, 0.05,
                                                         y_q=yq[j], want_deq=False)
                     for j in range(ncall)]
        elif kind == "i8q":
            xq = tq2.tq2_quantize_i8(xs, sc)  # once, outside the timed calls
            xqr = [xq.clone() for _ in range(ncall)]
            calls = [lambda j=j: tq2.tq2_gemv_i8q(copies[j][0][0], copies[j][0][1], xqr[j], sc, y=ys[j])
                     for j in range(ncall)]
        else:
            calls = [lambda j=j: tq2.tq2_gemv_i8(copies[j][0][0], copies[j][0][1], xr[j], sc, y=ys[j])
                     for j in range(ncall)]
        g = capture(torch, calls)
        time_graph(torch, g, WARM_REPLAYS)  # untimed: steady state before the timed replays
        ts = [time_graph(torch, g, 1) / ncall for _ in range(reps)]
        us, us95 = float(np.median(ts)), float(np.percentile(ts, 95))
        del g, calls, copies, xr, ys
        torch.cuda.empty_cache()

        rb = (sum(rows) * K * 66 // 256 + 255) // 256 * 256  # the call's weight bytes
        pool = torch.ones(ncopy * rb, dtype=torch.uint8, device="cuda")
        st = ctypes.c_void_p
        rcalls = [lambda j=j: probe.tq2probe_read(st(pool.data_ptr() + j * rb), rb, st(sink.data_ptr()), 2048,
                                                  st(torch.cuda.current_stream().cuda_stream))
                  for j in range(ncall)]
        g = capture(torch, rcalls)
        time_graph(torch, g, WARM_REPLAYS)
        us_rd = float(np.median([time_graph(torch, g, 1) / ncall for _ in range(reps)]))
        del g, rcalls, pool
        torch.cuda.empty_cache()
        gbs = nbytes / us / 1e3
        rd_gbs = rb / us_rd / 1e3
        if kind == "gemm16":
            nbytes_tok = nbytes
            gbs = nbytes / us / 1e3
            out[label] = {"us_per_call": round(us, 3), "us_per_call_p95": round(us95, 3),
                          "tokens_per_s": round(16e6 / us, 1),
                          "weight_GB_s": round(gbs, 1), "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
                          "read_probe_us": round(us_rd, 3),
                          "speedup_vs_16_gemv": None, "bytes_per_call": int(nbytes_tok),
                          "rotation_copies": ncopy}
            log(f"{label}: {us:.2f} us/call, {16e6 / us:.0f} tokens/s, weights at {gbs:.1f} GB/s")
            continue
        out[label] = {"us_per_call": round(us, 3), "us_per_call_p95": round(us95, 3), "GB_s": round(gbs, 1),
                      "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
                      "read_probe_us": round(us_rd, 3), "read_probe_GB_s": round(rd_gbs, 1),
                      "pct_of_read_probe": round(100 * gbs / rd_gbs, 1),
                      "bytes_per_call": int(nbytes), "rotation_copies": ncopy}
        log(f"{label}: {us:.2f} us/call, {gbs:.1f} GB/s ({gbs / PEAK_HBM_GBS:.1%}); "
            f"read probe {us_rd:.2f} us, {rd_gbs:.1f} GB/s")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg (and its parity gate)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--probes", action="store_true", help="also run the byte-counter calibration kernels")
    ap.add_argument("--no-configs", action="store_true", help="skip the single-call configuration timings")
    ap.add_argument("--config-calls", type=int, default=400,
                    help="calls per configuration graph (fewer for hardware-counter runs)")
    ap.add_argument("--config-reps", type=int, default=10, help="timed replays per configuration")
    ap.add_argument("--no-fused-step", action="store_true", help="skip the step built from the fused calls")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from ternary_packed_weight_amd import synth
    from ternary_packed_weight_amd import tq2

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    log(f"device: {torch.cuda.get_device_name(0)}; building the 224-linear stack")
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
    t_start = time.perf_counter()
    us_step = time_graph(torch, step_graph, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_bytes = sum(algo_bytes(e["N"], e["K"]) for e in stack)
    gbs = step_bytes / us_step / 1e3
    log(f"step: {us_step:.1f} us ({1e6 / us_step:.0f} steps/s), {gbs:.1f} GB/s; wall {wall:.3f} s")

    # ---- dominant kernel: the gate and up launches back to back
    dom = [e for e in stack if e["name"] in DOMINANT]
    dom_graph = capture(torch, [launch(e) for e in dom])
    time_graph(torch, dom_graph, 20)  # untimed warm-up replays
    us_dom = time_graph(torch, dom_graph, max(3, args.steps // 2)) / len(dom)
    dom_bytes = sum(algo_bytes(e["N"], e["K"]) for e in dom) / len(dom)
    achieved = dom_bytes / us_dom / 1e3
    sha = kernel_source_sha()
    traffic = traffic_from_profiles(sha)
    roofline = {"bound": "hbm", "kernel": DOMINANT_KERNEL,
                "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "bytes_per_launch": int(dom_bytes), "us_per_launch": round(us_dom, 3),
                "launches_timed": len(dom), "kernel_source_sha": sha}
    log(f"dominant kernel: {us_dom:.2f} us/launch, {achieved:.1f} GB/s ({achieved / PEAK_HBM_GBS:.1%})")

    step_fused = None if args.no_fused_step else fused_step(torch, tq2, stack, args.steps)

    if args.probes:
        # eager launches too, so per-dispatch counters see the dominant kernel
        for e in dom:
            launch(e)()
        torch.cuda.synchronize()
        run_probes(torch)

    configs = None
    if not args.no_configs:
        configs = time_configs(torch, tq2, synth, reps=args.config_reps, max_calls=args.config_calls)
        for label, rec in configs.items():
            if "speedup_vs_16_gemv" in rec:  # same shape as the gate/up launches timed above
                rec["speedup_vs_16_gemv"] = round(16 * us_dom / rec["us_per_call"], 2)
        # the fused q/k/v call against three single calls of its shapes (c1 for q, c0 for k and v)
        c0 = configs[CONFIGS[0][0]]["us_per_call"]
        c1 = configs[CONFIGS[1][0]]["us_per_call"]
        qkv = next(configs[label] for label, _, _, kind, _ in CONFIGS if kind == "qkv")
        qkv["three_single_calls_us"] = round(c1 + 2 * c0, 3)

    cpu, parity = None, None
    if not args.no_cpu:
        ys0 = [stack[i]["y"].cpu().numpy() for i in range(len(PROJ))]
        cpu, parity = cpu_leg(host_layer0, ys0, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads; parity {parity}")

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(us_step / 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "accumulate": "f32", "data": "synthetic",
        "config": {"workload": "MiniCPM4-8B decode step: 224 TQ2_0 linears (32 layers x q,k,v,o "
                               "4096/256/256/4096x4096, gate,up 16384x4096, down 4096x16384), fresh "
                               "fp16 x per linear, one stream, one HIP graph per step",
                   "bytes_per_step": step_bytes, "launches_per_step": len(stack),
                   "parallelism": "single GPU"},
        "steps_per_s": round(1e6 / us_step, 1),
        "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "roofline": roofline,
        "step_fused": step_fused,
        "configs": configs,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    if parity is not None and not parity["passed"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
