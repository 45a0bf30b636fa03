"""Benchmark of the Q4_0 decode GEMV / MoE decode / prefill GEMM kernels on one GPU.

Prints ONE JSON line on stdout (progress goes to stderr).

Headline workload (``value``): dense 7B-shaped decode linears, Q4_0 weights
4096x4096 (attention projection), 4096x11008 twice (gate, up) and 11008x4096
(down), each at batch 1, 4 and 8 -> one step = 12 q4_0_gemv calls. ``value``
is the step's algorithmic HBM bytes (each Q4_0 block once at 18 B per 32
weights, plus activations and outputs) divided by the step time, in GB/s.
Weights rotate over enough identical copies (>= 1 GiB in total) that every
step reads them from HBM rather than from the 256 MB Infinity Cache.

Also measured in the same run (reported under "also"): the DeepSeek-V2-shaped
MoE decode (5120 hidden, 160 experts of 5120x1536 gate/up and 1536x5120 down,
top-6) at 1 and 32 tokens (uniform and skewed routing) in tokens/s and GB/s,
and the prefill GEMM 2048x4096 . 4096x{4096, 11008} in TFLOP/s.

Attainable roofs (``also.probes``, from libq4probe.so): a read-only 16-byte
stream at the byte counts of the decode calls and at 1 GiB, and fp16 / fp32
MFMA loops; every per-call rate is also given as a fraction of the stream
rate at its size.

``cpu_baseline``: the CPU oracle (single-threaded, double accumulation) pinned
to one host core, on bounded samples of every workload (dense steps in GB/s;
MoE decode in tokens/s; prefill rows in TFLOP/s), about 20 s in all. A
reported baseline, not a target.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s
VALU_F32_PEAK_TFLOPS = 78.6    # 256 CU x 4 SIMD x 16 lanes x 2.4 GHz x 2 flop (no packed FP32)
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA, TFLOP/s
GIB = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def q4_bytes(K, N):
    return K * (N // 32) * 18


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the pinned single-core oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the MoE and prefill measurements")
    ap.add_argument("--only", choices=["dense", "moe", "prefill", "probes", "traffic-probe"],
                    default=None,
                    help="run a single workload (for profiling); prints its own JSON line")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write the HBM traffic summary from two counter passes of the probe")
    return ap.parse_args()


class EventTimer:
    """Durations from HIP events recorded on the launching stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, key, fn):
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.pairs.setdefault(key, []).append((s, e))
        return out

    def mean_ms(self, key):
        ps = self.pairs.get(key, [])
        return sum(s.elapsed_time(e) for s, e in ps) / len(ps) if ps else float("nan")


def capture(torch, fn):
    """Capture fn's kernel launches (made on the current stream) into a HIP graph."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(torch, graphs, reps):
    """Total seconds of `reps` round-robin replays, with events only around all
    of them: an event recorded between two replays adds a gap of its own (about
    5 us per replay on MI355X), so it stays out of the mean."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        graphs[r % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3


def time_graph_dist(torch, graphs, reps, per_replay):
    """Replay the graphs round robin; each replay holds `per_replay` units
    (steps or launches). Returns the mean time per unit, from a pass with events
    only around all replays, and the per-replay times per unit, from a pass
    before it with an event after every replay (those include the events' own
    gaps, so their quantiles sit a few microseconds per replay above the mean;
    the pass also warms the clocks up for the mean's)."""
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record()
    for r in range(reps):
        graphs[r % len(graphs)].replay()
        evs[r + 1].record()
    torch.cuda.synchronize()
    ts = [evs[r].elapsed_time(evs[r + 1]) * 1e-3 / per_replay for r in range(reps)]
    mean = time_replays(torch, graphs, reps) / (reps * per_replay)
    return mean, ts


def time_graph(torch, graphs, reps, per_replay):
    """Mean time per unit of work over `reps` round-robin replays."""
    return time_graph_dist(torch, graphs, reps, per_replay)[0]


MOE_CALLS_PER_GRAPH = 8


def time_calls(torch, call, reps):
    """Per-call time of call(r), r = 0, 1, ...: 16 graphs of MOE_CALLS_PER_GRAPH
    consecutive calls each (graph c holds calls 8c .. 8c + 7, so the layer copies
    and routings rotate inside a graph as they do across graphs), replayed round
    robin. A decode step's graph holds the MoE call of every layer, so a graph
    replay's own start-up cost is shared by many calls there; timing one call per
    graph instead adds that cost (about 4 us on MI355X) to every call. The one-call
    figure is returned too. Returns (mean s, per-replay s per call, one-call mean s)."""
    G = MOE_CALLS_PER_GRAPH
    graphs = [capture(torch, lambda c=c: [call(c * G + u) for u in range(G)]) for c in range(16)]
    dt, ts = time_graph_dist(torch, graphs, reps, G)
    del graphs
    g1 = [capture(torch, lambda r=r: call(r)) for r in range(16)]
    dt1, _ = time_graph_dist(torch, g1, reps, 1)
    return dt, ts, dt1


def quantiles_us(ts):
    """p10, median and p90 of a list of durations (seconds), in microseconds."""
    v = sorted(ts)
    q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))] * 1e6
    return {"p10_us": round(q(0.1), 2), "median_us": round(q(0.5), 2), "p90_us": round(q(0.9), 2),
            "n": len(v)}


# ---------------------------------------------------------------------------
# dense decode linears
# ---------------------------------------------------------------------------
def bench_dense(torch, dev, steps, warmup):
    from moe_experts_amd import datagen, q4_0_gemv, q4_0_gemv_workspace_bytes
    shapes = datagen.DENSE_7B_SHAPES
    Ms = datagen.DENSE_7B_BATCHES
    wbytes = sum(q4_bytes(K, N) for _, K, N, _ in shapes)
    R = max(2, math.ceil(GIB / wbytes))
    log(f"[dense] generating 4 matrices ({wbytes / 1e6:.1f} MB), {R} device copies")
    host = [datagen.q4_0_random(seed, K, N) for _, K, N, seed in shapes]
    base = [torch.from_numpy(h).to(dev) for h in host]
    copies = [base] + [[b.clone() for b in base] for _ in range(R - 1)]
    xs = {M: {K: torch.from_numpy(datagen.activations(datagen.dense_x_seed(M), M, K)).to(dev)
              for K in sorted({K for _, K, _, _ in shapes})} for M in Ms}
    ys = {(M, i): torch.empty((M, N), dtype=torch.float32, device=dev)
          for M in Ms for i, (_, _, N, _) in enumerate(shapes)}

    need = max(q4_0_gemv_workspace_bytes(M, N, K) for M in Ms for _, K, N, _ in shapes)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    calls = [(M, i) for M in Ms for i in range(len(shapes))]
    step_bytes = sum(q4_bytes(K, N) + 4 * M * K + 4 * M * N
                     for M in Ms for _, K, N, _ in shapes)

    def step(r):
        w = copies[r % R]
        for (M, i) in calls:
            _, K, N, _ = shapes[i]
            q4_0_gemv(xs[M][K], w[i], N, y=ys[(M, i)], ws=ws)

    # one HIP graph per weight copy, each holding one whole step (12 GEMVs);
    # replaying them round robin keeps the host out of the timed region
    for r in range(warmup):
        step(r)
    graphs = [capture(torch, lambda r=r: step(r)) for r in range(R)]
    for r in range(warmup):
        graphs[r % R].replay()
    torch.cuda.synchronize()
    # the timed steps: events only before the first and after the last
    order = [graphs[(warmup + r) % R] for r in range(R)]
    t0 = time.perf_counter()
    dt = time_replays(torch, order, steps) / steps
    wall = (time.perf_counter() - t0) / steps
    # the distribution, from the same steps again with an event after each
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for r in range(steps):
        order[r % R].replay()
        evs[r + 1].record()
    torch.cuda.synchronize()
    step_dist = quantiles_us([evs[r].elapsed_time(evs[r + 1]) * 1e-3 for r in range(steps)])

    # per call: graphs of 8 back-to-back launches of each call. Each matrix gets
    # its own rotation of at least 1 GiB of copies (the step's copies plus
    # clones), and the graphs walk through all of them, so every launch reads
    # its weights from HBM rather than from the 256 MB Infinity Cache.
    per_call, per_M, call_s = {}, {}, {}
    rot = []
    for i, (_, K, N, _) in enumerate(shapes):
        Ri = max(16, math.ceil(GIB / q4_bytes(K, N)))
        Ri = (Ri + 7) // 8 * 8
        rot.append([copies[r][i] for r in range(R)] + [base[i].clone() for _ in range(Ri - R)])
    for (M, i) in calls:
        name, K, N, _ = shapes[i]
        ng = len(rot[i]) // 8
        gs = [capture(torch, lambda c=c: [q4_0_gemv(xs[M][K], rot[i][c * 8 + u], N,
                                                    y=ys[(M, i)], ws=ws) for u in range(8)])
              for c in range(ng)]
        t, ts = time_graph_dist(torch, gs, max(4 * ng, 48), 8)
        call_s[(M, i)] = t
        b = q4_bytes(K, N) + 4 * M * K + 4 * M * N
        per_call[f"{name}_M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1),
                                    "TFLOPs": round(2 * M * K * N / t / 1e12, 2),
                                    "bytes": b, **quantiles_us(ts)}
        del gs
    for M in Ms:
        t = sum(call_s[(M, i)] for i in range(len(shapes)))
        b = sum(q4_bytes(K, N) + 4 * M * K + 4 * M * N for _, K, N, _ in shapes)
        per_M[M] = (t * 1e3, b)
    del rot
    return dict(step_s=dt, wall_s=wall, step_bytes=step_bytes, per_call=per_call, per_M=per_M,
                call_s=call_s, step_dist=step_dist,
                R=R, host=host, shapes=shapes, Ms=Ms)


def bench_q8(torch, dev, steps, warmup, d):
    """q8_0_gemv on the dense 7B shapes at batch 1 and 8 (Q8_0 weights: 34 bytes
    per 32 weights), timed like the Q4_0 calls, and the batch-1 token-rate ratio
    Q8_0 / Q4_0 over the four matrices (the article's CPU figure is about 60 %)."""
    from moe_experts_amd import datagen, q8_0_gemv, q8_0_gemv_workspace_bytes
    shapes = datagen.DENSE_7B_SHAPES
    q8b = lambda K, N: K * (N // 32) * 34
    wbytes = sum(q8b(K, N) for _, K, N, _ in shapes)
    R = max(2, math.ceil(GIB / wbytes))
    base = [torch.from_numpy(datagen.q8_0_random(seed + 4000, K, N)).to(dev)
            for _, K, N, seed in shapes]
    copies = [base] + [[b.clone() for b in base] for _ in range(R - 1)]
    need = max(q8_0_gemv_workspace_bytes(M, N, K) for M in (1, 8) for _, K, N, _ in shapes)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    res, t8 = {}, {}
    for M in (1, 8):
        for i, (name, K, N, _) in enumerate(shapes):
            x = torch.from_numpy(datagen.activations(datagen.dense_x_seed(M), M, K)).to(dev)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            for u in range(warmup):
                q8_0_gemv(x, copies[u % R][i], N, y=y, ws=ws)
            gs = [capture(torch, lambda c=c: [q8_0_gemv(x, copies[(c * 8 + u) % R][i], N, y=y,
                                                        ws=ws) for u in range(8)])
                  for c in range(2)]
            t = time_graph(torch, gs, max(steps, 10), 8)
            t8[(M, i)] = t
            b = q8b(K, N) + 4 * M * K + 4 * M * N
            res[f"{name}_M{M}"] = {"us": round(t * 1e6, 2), "GBps": round(b / t / 1e9, 1)}
    q4_t = sum(d["call_s"][(1, i)] for i in range(len(shapes)))
    q8_t = sum(t8[(1, i)] for i in range(len(shapes)))
    res["token_rate_vs_q4_0_M1"] = round(q4_t / q8_t, 3)
    log(f"[q8_0] {res}")
    return res


# The dominant unit of the headline step: q4_0_gemv at batch 8 on the
# 4096 x 11008 gate matrix. Batch 8 takes the largest share of the step, and
# its gate, up and down calls are the longest launches. One call is two
# dispatches: the matrix-core kernel gemv_q4_0_mfma_kernel<2,8,4> and its
# split-K reduce kernel.
DOMINANT = {"M": 8, "shape": "ffn_gate"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_q4_0_M8_4096x11008_traffic.md")
MAIN_KERNEL = "gemv_q4_0_mfma_kernel"
KERNEL_SOURCES = ["moe_experts_amd/csrc/q4_device.hpp", "moe_experts_amd/csrc/q4_mfma.hpp",
                  "moe_experts_amd/csrc/gemv_q4_0.hip", "moe_experts_amd/csrc/gemv_mfma_q4_0.hip",
                  "moe_experts_amd/csrc/q4moe_api.cpp", "moe_experts_amd/build.py"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per call of the dominant unit from the committed counter
    summary, or None when it is missing or was taken on other kernel code."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    blob = json.loads(text[start + 7:text.index("```", start + 7)])
    if blob.get("source_hash") != kernel_source_hash():
        return None
    return blob.get("hbm_bytes_per_call")


def dense_roofline(d, probes):
    """Roofline of the dominant unit (see DOMINANT).

    The batch-8 call runs on the fp32 matrix cores: every weight is one
    multiply-add per activation row, 2MKN flops in all, done by
    v_mfma_f32_4x4x1 (4 activation rows per instruction, no padding at batch 8).
    The vector ALU unpacks the nibbles: per row of 16 MFMA blocks (512
    weights) each lane issues about 17 instructions (2 masks, 8 converts, the
    scale convert, products and corrections, 2 offsets). Within one wave the
    matrix and vector instructions issue one after the other (a one-wave probe:
    adding the unpack work lowered the MFMA rate by its own issue time); the
    two waves of a SIMD overlap them (each batch converts first, then issues its
    MFMAs). So the issue floor lies between the larger of the two (overlapped)
    and their sum (serial); both are reported."""
    M = DOMINANT["M"]
    shapes = d["shapes"]
    i = [k for k, sh in enumerate(shapes) if sh[0] == DOMINANT["shape"]][0]
    _, K, N, _ = shapes[i]
    t = d["call_s"][(M, i)]
    flops = 2 * M * K * N
    algo_bytes = q4_bytes(K, N) + 4 * M * K + 4 * M * N
    mfma_flops = 2 * (4 * ((M + 3) // 4)) * K * N  # the instruction's 4-row granularity
    mfma_s = mfma_flops / (MFMA_F32_PEAK_TFLOPS * 1e12)
    valu_lane_ops = K * N * 17.0 * 64 / 512
    valu_s = valu_lane_ops / (VALU_F32_PEAK_TFLOPS * 1e12 / 2)
    hbm_s = algo_bytes / (HBM_PEAK_GBS * 1e9)
    tflops = flops / t / 1e12
    gbs = algo_bytes / t / 1e9
    roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": MFMA_F32_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            "kernel": f"q4_0_gemv M={M} on 4096x11008 (gemv_q4_0_mfma_kernel<2,8,4> + "
                      "gemv_reduce_kernel)",
            "avg_launch_us": round(t * 1e6, 2),
            "algorithmic_bytes": algo_bytes, "algorithmic_flops": flops,
            "mfma_bound_us": round(mfma_s * 1e6, 2), "hbm_bound_us": round(hbm_s * 1e6, 2),
            "issue_bound_us": round((mfma_s + valu_s) * 1e6, 2),
            "issue_frac": round((mfma_s + valu_s) / t, 4),
            "overlapped_issue_bound_us": round(max(mfma_s, valu_s) * 1e6, 2),
            "hbm_GBps": round(gbs, 1),
            "attainable_GBps": attainable_for(probes, algo_bytes),
            "attainable_frac": round(gbs / attainable_for(probes, algo_bytes), 4),
            "attainable_mfma_f32_TFLOPs": probes["mfma_f32_TFLOPs"],
            "attainable_mfma_frac": round(tflops / probes["mfma_f32_TFLOPs"], 4),
            "note": "achieved = 2MKN / call time against the fp32 MFMA peak; issue_bound adds "
                    "the vector unpack work to the MFMA time (serial within a wave), "
                    "overlapped_issue_bound takes the larger of the two (two waves per SIMD "
                    "overlap them)"}
    return roof


def traffic_probe(torch, dev):
    """Workload for the FETCH_SIZE / WRITE_SIZE counter passes: 24 calls of the
    dominant unit on rotating weight copies, then 4 device copies of a known
    512 MiB buffer (calibration: bytes the counter reports for a plain copy)."""
    from moe_experts_amd import datagen, q4_0_gemv
    M = DOMINANT["M"]
    name, K, N, seed = [sh for sh in datagen.DENSE_7B_SHAPES if sh[0] == DOMINANT["shape"]][0]
    B0 = torch.from_numpy(datagen.q4_0_random(seed, K, N)).to(dev)
    copies = [B0] + [B0.clone() for _ in range(max(2, math.ceil(GIB / B0.numel())) - 1)]
    x = torch.from_numpy(datagen.activations(datagen.dense_x_seed(M), M, K)).to(dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    for r in range(24):
        q4_0_gemv(x, copies[r % len(copies)], N, y=y)
    torch.cuda.synchronize()
    del copies
    src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "traffic", "calls": 24, "copy_bytes": src.numel()}), flush=True)


def traffic_summary(fetch_csv, write_csv, command):
    """Turn the two counter passes of traffic_probe into TRAFFIC_FILE."""
    import csv

    def per_kernel(path, counter):
        out = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]) * 1024.0)
        return out

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = 512 << 20

    def pick(d, key):
        ks = [k for k in d if key in k]
        if not ks:
            raise SystemExit(f"no dispatch of {key} in the counter file")
        return d[ks[0]]

    def med(v):
        v = sorted(v)
        return v[len(v) // 2]

    # the probe's last four copies are the 512 MiB calibration copies (earlier
    # copy dispatches clone the weight matrix)
    cf = med(pick(fetch, "copyBuffer")[-4:])
    cw = med(pick(write, "copyBuffer")[-4:])
    f_fetch = copy_bytes / cf
    f_write = copy_bytes / cw
    main_f = med(pick(fetch, MAIN_KERNEL)[4:])
    main_w = med(pick(write, MAIN_KERNEL)[4:])
    red_f = med(pick(fetch, "gemv_reduce_kernel")[4:])
    red_w = med(pick(write, "gemv_reduce_kernel")[4:])
    M = DOMINANT["M"]
    K, N = 4096, 11008
    algo = q4_bytes(K, N) + 4 * M * K + 4 * M * N
    total = (main_f + red_f) * f_fetch + (main_w + red_w) * f_write
    blob = {"source_hash": kernel_source_hash(), "hbm_bytes_per_call": round(total),
            "algorithmic_bytes_per_call": algo,
            "main_kernel": {"fetch_bytes": round(main_f * f_fetch), "write_bytes": round(main_w * f_write)},
            "reduce_kernel": {"fetch_bytes": round(red_f * f_fetch), "write_bytes": round(red_w * f_write)},
            "calibration": {"copy_bytes": copy_bytes, "fetch_counter_bytes": round(cf),
                            "write_counter_bytes": round(cw), "fetch_factor": round(f_fetch, 4),
                            "write_factor": round(f_write, 4)}}
    text = f"""# HBM traffic of q4_0_gemv, batch 8, 4096 x 11008 (gate shape of the dense decode step)

Counters: `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch, rocprofv3 `--pmc`), one pass each,
over the workload of `python bench.py --only traffic-probe` (24 calls on rotating weight copies,
then 4 device copies of 512 MiB). Median over the calls after the first four.

Calibration: a plain 512 MiB device copy reads {cf / 2**20:.1f} MiB by `FETCH_SIZE` and writes
{cw / 2**20:.1f} MiB by `WRITE_SIZE`; the factors {f_fetch:.4f} (fetch) and {f_write:.4f} (write)
scale the kernel's counter values to bytes.

| dispatch | fetched (B) | written (B) |
|---|---|---|
| gemv_q4_0_mfma_kernel<2,8,4> | {round(main_f * f_fetch)} | {round(main_w * f_write)} |
| gemv_reduce_kernel | {round(red_f * f_fetch)} | {round(red_w * f_write)} |
| **call** | {round((main_f + red_f) * f_fetch)} | {round((main_w + red_w) * f_write)} |

Algorithmic bytes per call: {algo} (weights once, activations, outputs). Measured / algorithmic:
{total / algo:.3f}.

Commands:
```
{command}
```

```json
{json.dumps(blob, indent=1)}
```
"""
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write(text)
    print(text)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baselines(d, seconds):
    """The oracle as it stands (single-threaded C++, double accumulation),
    pinned to one host core in this process, on bounded samples of each
    workload: whole dense decode steps (GB/s of the same algorithmic bytes),
    the single-token MoE decode and four tokens of the 32-token batch
    (tokens/s), and 32 rows of the 2048 x 4096 x 4096 prefill (TFLOP/s)."""
    import oracle
    from moe_experts_amd import datagen
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})
    try:
        out = {}
        # dense decode step
        shapes, Ms = d["shapes"], d["Ms"]
        xs = {M: {K: datagen_x(M, K) for K in sorted({K for _, K, _, _ in shapes})} for M in Ms}
        done, t0, nsteps = 0, time.perf_counter(), 0
        while True:
            for M in Ms:
                for i, (_, K, N, _) in enumerate(shapes):
                    oracle.q4_0_matmul(xs[M][K], d["host"][i], N, K, with_bound=False)
                    done += q4_bytes(K, N) + 4 * M * K + 4 * M * N
            nsteps += 1
            if time.perf_counter() - t0 >= 0.4 * seconds:
                break
        dt = time.perf_counter() - t0
        out["dense_GBps"] = round(done / dt / 1e9, 4)
        dense_sample = f"{nsteps} dense step(s) in {dt:.1f} s"
        # MoE decode: one token, and 4 tokens of the 32-token batch
        c = datagen.MOE_DSV2
        H, I, E, topk = c["H"], c["I"], c["E"], c["topk"]
        for label, T, cfg, ntok in (("moe_t1", 1, datagen.MOE_T1, 1),
                                    ("moe_t32", 32, datagen.MOE_T32, 4)):
            x = datagen.activations(cfg["x_seed"], T, H)[:ntok]
            ids, w, _ = datagen.routing(cfg["logit_seed"], T, E, topk)
            ids, w = ids[:ntok], w[:ntok]
            Wg, Wu, Wd = datagen.moe_experts(H, I, E, experts=sorted(set(ids.ravel().tolist())))
            calls, t0 = 0, time.perf_counter()
            while True:
                oracle.moe_decode(x, Wg, Wu, Wd, ids, w, H, I, E, with_bound=False)
                calls += 1
                if time.perf_counter() - t0 >= 0.15 * seconds:
                    break
            dt = time.perf_counter() - t0
            out[f"{label}_tokens_per_s"] = round(calls * ntok / dt, 3)
            del Wg, Wu, Wd
        # prefill GEMM rows
        pc = datagen.PREFILL
        K, N = pc["K"], pc["Ns"][0]
        X16 = datagen.to_f16(datagen.activations(pc["x_seed"], 32, K))
        B = datagen.q4_0_random(pc["b_seeds"][0], K, N)
        calls, t0 = 0, time.perf_counter()
        while True:
            oracle.q4_0_matmul_f16(X16, B, N, K, with_bound=False)
            calls += 1
            if time.perf_counter() - t0 >= 0.15 * seconds:
                break
        dt = time.perf_counter() - t0
        out["prefill_TFLOPs"] = round(calls * 2 * 32 * K * N / dt / 1e12, 6)
    finally:
        os.sched_setaffinity(0, set(allowed))
    return {"value": out["dense_GBps"], "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{dense_sample} (12 GEMVs each); MoE: repeated single-token and 4-token "
                      "calls of the decode configurations; prefill: 32 rows of 2048 x 4096 x "
                      "4096; single thread pinned to one core, double accumulation",
            "cpu": cpu_model(), "pinned_core": core, "logical_cpus": os.cpu_count(),
            "per_config": out}


def datagen_x(M, K):
    from moe_experts_amd import datagen
    return datagen.activations(datagen.dense_x_seed(M), M, K)


# ---------------------------------------------------------------------------
# attainable roofs (libq4probe.so)
# ---------------------------------------------------------------------------
# Byte counts of the read-only stream probe: the algorithmic bytes of the
# 4096 x 4096 call at batch 1, of a 4096 x 11008 call at batch 1, of the
# six routed experts of a single-token MoE decode, and 1 GiB.
PROBE_SIZES = {"gemv_4096x4096": 9469952, "gemv_4096x11008": 25422848,
               "moe_t1_experts": 79626240, "1GiB": GIB}


def bench_probes(torch, dev):
    """Attainable rates measured with the probes: a read-only 16-byte stream at
    the byte counts of the decode calls (each launch reads a different region
    of a 2 GiB buffer, so the rotation spans far more than the 256 MB Infinity
    Cache), best over grids of 256..2048 workgroups; and fp16 / fp32 MFMA
    loops (4 waves per SIMD)."""
    from moe_experts_amd import probe
    span = 2 * GIB
    buf = torch.empty(span + (1 << 20), dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    res = {"stream": {}}
    for name, nbytes in PROBE_SIZES.items():
        stride = (nbytes + 4095) // 4096 * 4096
        nreg = max(1, span // stride)
        per = min(nreg, 64)
        best = None
        for grid in (256, 512, 1024, 2048):
            def run(c, grid=grid):
                for u in range(per):
                    probe.stream_read(buf, ((c * per + u) % nreg) * stride, nbytes, grid, sink)
            gs = [capture(torch, lambda c=c: run(c)) for c in range(max(1, min(4, nreg // per)))]
            t, ts = time_graph_dist(torch, gs, 8 if nbytes < GIB else 4, per)
            if best is None or t < best[0]:
                best = (t, grid, ts)
        t, grid, ts = best
        res["stream"][name] = {"bytes": nbytes, "us": round(t * 1e6, 2),
                               "GBps": round(nbytes / t / 1e9, 1), "grid": grid}
        log(f"[probe] stream {name}: {res['stream'][name]}")
    # The decode GEMV's access pattern: the same matrices read as split-K
    # tiles, at the batch-1 plan's tile (16 blocks x Kt rows) and at small
    # tiles (32 blocks x about 40 rows, about 1024 workgroups).
    from moe_experts_amd import datagen, q4_0_gemv_workspace_bytes
    res["tile"] = {}
    for name, K, N, _seed in datagen.DENSE_7B_SHAPES:
        if name == "ffn_up":
            continue
        pitch = N // 32 * 18
        nbytes = K * pitch
        stride = (nbytes + 4095) // 4096 * 4096
        nreg = max(1, span // stride)
        per = min(nreg, 64)
        S = max(1, q4_0_gemv_workspace_bytes(1, N, K) // (4 * N))
        for label, seg, kt in (("plan_m1", 288, -(-K // S)), ("small", 576, -(-K // max(1, 1024 // -(-pitch // 576))))):
            def run(c, seg=seg, kt=kt):
                for u in range(per):
                    probe.tile_read(buf, ((c * per + u) % nreg) * stride, K, pitch, seg, kt, sink)
            gs = [capture(torch, lambda c=c: run(c)) for c in range(max(1, min(4, nreg // per)))]
            t, _ = time_graph_dist(torch, gs, 8, per)
            grid = -(-pitch // seg) * -(-K // kt)
            res["tile"][f"{name}_{label}"] = {"bytes": nbytes, "seg": seg, "kt": kt, "grid": grid,
                                              "us": round(t * 1e6, 2),
                                              "GBps": round(nbytes / t / 1e9, 1)}
            log(f"[probe] tile {name} {label}: {res['tile'][f'{name}_{label}']}")
    # A kernel boundary: empty kernels back to back, and a stream of the 4096 x
    # 4096 matrix's bytes with and without an empty kernel after each read.
    nb = PROBE_SIZES["gemv_4096x4096"]
    stride = (nb + 4095) // 4096 * 4096
    nreg = span // stride
    g_empty = capture(torch, lambda: [probe.empty(sink) for _ in range(64)])
    t_empty = time_graph(torch, [g_empty], 8, 64)
    per = 64

    def reads(c, with_empty):
        for u in range(per):
            probe.stream_read(buf, ((c * per + u) % nreg) * stride, nb, 1024, sink)
            if with_empty:
                probe.empty(sink)
    t_plain = time_graph(torch, [capture(torch, lambda c=c: reads(c, False)) for c in range(2)], 8, per)
    t_pair = time_graph(torch, [capture(torch, lambda c=c: reads(c, True)) for c in range(2)], 8, per)
    res["kernel_boundary"] = {"empty_kernel_us": round(t_empty * 1e6, 2),
                              "stream_9.47MB_us": round(t_plain * 1e6, 2),
                              "stream_then_empty_us": round(t_pair * 1e6, 2),
                              "added_by_empty_us": round((t_pair - t_plain) * 1e6, 2)}
    log(f"[probe] kernel boundary: {res['kernel_boundary']}")
    del buf
    msink = torch.zeros(1024 * 256, dtype=torch.float32, device=dev)
    for kind, iters in (("f16", 4096), ("f32", 8192)):
        flops = [0]

        def run(kind=kind, iters=iters):
            flops[0] = probe.mfma_loop(kind, iters, 1024, msink)
        g = capture(torch, lambda: [run() for _ in range(4)])
        t = time_graph(torch, [g], 8, 4)
        res[f"mfma_{kind}_TFLOPs"] = round(flops[0] / t / 1e12, 1)
        log(f"[probe] mfma {kind}: {res[f'mfma_{kind}_TFLOPs']} TFLOP/s")
    return res


def attainable_for(probes, nbytes):
    """The stream probe rate measured at the probe size closest to nbytes."""
    st = probes["stream"]
    k = min((k for k in st if k != "1GiB"), key=lambda k: abs(math.log(st[k]["bytes"] / nbytes)))
    return st[k]["GBps"]


# ---------------------------------------------------------------------------
# MoE decode
# ---------------------------------------------------------------------------
def bench_moe(torch, dev, steps, warmup):
    from moe_experts_amd import datagen, moe_q4_0_decode, moe_q4_0_workspace_bytes
    c, L = datagen.MOE_DSV2, datagen.MOE_LAYER
    H, I, E, topk = c["H"], c["I"], c["E"], c["topk"]
    Es = E + L["n_shared"]
    log(f"[moe] generating {Es} experts ({E} routed, {L['n_shared']} shared; 2.15 GB)")
    Wg, Wu, Wd = datagen.moe_experts(H, I, Es)
    layers = 4  # distinct copies of the layer, visited round robin (>8 GB)
    dW = [(torch.from_numpy(Wg).to(dev), torch.from_numpy(Wu).to(dev), torch.from_numpy(Wd).to(dev))]
    for _ in range(layers - 1):
        dW.append(tuple(w.clone() for w in dW[0]))
    del Wg, Wu, Wd
    routed = [tuple(w[:E] for w in ws) for ws in dW]  # the decode alone: routed experts only
    mat = H * (I // 32) * 18
    res = {}
    for label, T, bias, xseed, lseed in (("t1", 1, 0.0, datagen.MOE_T1["x_seed"], datagen.MOE_T1["logit_seed"]),
                                         ("t32", 32, 0.0, datagen.MOE_T32["x_seed"], datagen.MOE_T32["logit_seed"]),
                                         ("t32_skewed", 32, datagen.MOE_T32["hot_bias"],
                                          datagen.MOE_T32["x_seed"], datagen.MOE_T32["logit_seed"])):
        x = torch.from_numpy(datagen.activations(xseed, T, H)).to(dev)
        routes = []
        uniq = []
        for r in range(16):
            ids, w, _ = datagen.routing(lseed + 1000 * r, T, E, topk, hot_bias=bias)
            routes.append((torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)))
            uniq.append(len(np.unique(ids)))
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = torch.zeros(moe_q4_0_workspace_bytes(T, H, I, E, topk), dtype=torch.uint8, device=dev)

        def call(r):
            g, u, dd = routed[r % layers]
            ids, w = routes[r % len(routes)]
            moe_q4_0_decode(x, g, u, dd, ids, w, I, E, out=out, ws=ws)

        for r in range(warmup):
            call(r)
        dt, ts, dt1 = time_calls(torch, call, max(steps, 64))
        U = np.mean([uniq[r % len(routes)] for r in range(16)])
        b = U * 3 * mat + 2 * 4 * T * H + T * topk * 8
        res[label] = {"tokens_per_s": round(T / dt, 1), "us_per_call": round(dt * 1e6, 2),
                      "GBps": round(b / dt / 1e9, 1), "hbm_frac": round(b / dt / 1e9 / HBM_PEAK_GBS, 4),
                      "unique_experts": round(float(U), 2), **quantiles_us(ts),
                      "us_per_call_graph1": round(dt1 * 1e6, 2)}
        log(f"[moe] {label}: {res[label]}")
    res.update(bench_moe_layer(torch, dev, steps, warmup, dW))
    res.update(bench_moe_prefill(torch, dev, steps, warmup, routed))
    return res


def bench_moe_prefill(torch, dev, steps, warmup, routed):
    """moe_q4_0_prefill: 2048 prompt tokens, top-6 of the 160 routed experts
    (uniform routing), experts as grouped GEMMs on the fp16 matrix cores.
    Useful flops: 3 products of 2*H*I per valid (token, slot) pair."""
    from moe_experts_amd import datagen, moe_q4_0_prefill, moe_q4_0_prefill_workspace_bytes
    c = datagen.MOE_DSV2
    H, I, E, topk = c["H"], c["I"], c["E"], c["topk"]
    T = 2048
    x16 = torch.from_numpy(datagen.to_f16(datagen.activations(5101, T, H))).to(dev)
    routes = []
    for r in range(4):
        ids, w, _ = datagen.routing(5301 + 1000 * r, T, E, topk)
        routes.append((torch.from_numpy(ids).to(dev), torch.from_numpy(w).to(dev)))
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(moe_q4_0_prefill_workspace_bytes(T, H, I, E, topk), dtype=torch.uint8,
                     device=dev)
    layers = len(routed)

    def call(r):
        g, u, dd = routed[r % layers]
        ids, w = routes[r % len(routes)]
        moe_q4_0_prefill(x16, g, u, dd, ids, w, I, E, out=out, ws=ws)

    for r in range(warmup):
        call(r)
    graphs = [capture(torch, lambda r=r: call(r)) for r in range(4)]
    dt, ts = time_graph_dist(torch, graphs, max(steps // 2, 16), 1)
    flops = T * topk * 3 * 2.0 * H * I
    tf = flops / dt / 1e12
    res = {"prefill_t2048": {"tokens_per_s": round(T / dt, 1), "us_per_call": round(dt * 1e6, 1),
                             "TFLOPs": round(tf, 1), "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                             **quantiles_us(ts)}}
    log(f"[moe] prefill_t2048: {res['prefill_t2048']}")
    return res


def bench_moe_layer(torch, dev, steps, warmup, dW):
    """Whole layer (moe_q4_0_layer): the on-device router, then the routed and
    shared experts. The routing comes from the router, so each call's x differs
    (16 seeds) and the unique experts are counted from the router's own ids."""
    from moe_experts_amd import (datagen, moe_q4_0_layer, moe_q4_0_layer_workspace_bytes,
                                 moe_router_topk)
    c, L = datagen.MOE_DSV2, datagen.MOE_LAYER
    H, I, E, topk, ns = c["H"], c["I"], c["E"], c["topk"], L["n_shared"]
    layers = len(dW)
    Wr0 = torch.from_numpy(datagen.router_weights(L["router_seed"], E, H)).to(dev)
    Wr = [Wr0] + [Wr0.clone() for _ in range(layers - 1)]  # one router per layer copy
    mat = H * (I // 32) * 18
    res = {}
    for label, T, xseed in (("layer_t1", 1, datagen.MOE_T1["x_seed"]),
                            ("layer_t32", 32, datagen.MOE_T32["x_seed"])):
        xs = [torch.from_numpy(datagen.activations(xseed + 1000 * r, T, H)).to(dev)
              for r in range(16)]
        uniq = []
        for x in xs:
            ids = moe_router_topk(x, Wr0, topk, ns)[1].cpu().numpy()
            uniq.append(len(np.unique(ids[:, :topk][ids[:, :topk] >= 0])) + ns)
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = torch.zeros(moe_q4_0_layer_workspace_bytes(T, H, I, E, topk, ns), dtype=torch.uint8,
                         device=dev)

        def call(r):
            g, u, dd = dW[r % layers]
            moe_q4_0_layer(xs[r % 16], Wr[r % layers], g, u, dd, I, topk, ns, out=out, ws=ws)

        for r in range(warmup):
            call(r)
        dt, ts, dt1 = time_calls(torch, call, max(steps, 64))
        U = float(np.mean(uniq))
        b = U * 3 * mat + E * H * 4 + 2 * 4 * T * H
        res[label] = {"tokens_per_s": round(T / dt, 1), "us_per_call": round(dt * 1e6, 2),
                      "GBps": round(b / dt / 1e9, 1), "hbm_frac": round(b / dt / 1e9 / HBM_PEAK_GBS, 4),
                      "unique_experts_incl_shared": round(U, 2), **quantiles_us(ts),
                      "us_per_call_graph1": round(dt1 * 1e6, 2)}
        log(f"[moe] {label}: {res[label]}")
    return res


# ---------------------------------------------------------------------------
# prefill GEMM
# ---------------------------------------------------------------------------
def bench_prefill(torch, dev, steps, warmup):
    from moe_experts_amd import datagen, q4_0_gemm
    c = datagen.PREFILL
    M, K = c["M"], c["K"]
    X = torch.from_numpy(datagen.to_f16(datagen.activations(c["x_seed"], M, K))).to(dev)
    res = {}
    for N, seed in zip(c["Ns"], c["b_seeds"]):
        B = torch.from_numpy(datagen.q4_0_random(seed, K, N)).to(dev)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        for _ in range(warmup):
            q4_0_gemm(X, B, N, Y=Y)
        g = capture(torch, lambda: [q4_0_gemm(X, B, N, Y=Y) for _ in range(4)])
        t, ts = time_graph_dist(torch, [g], max(steps, 64) // 4 + 1, 4)
        ms = t * 1e3
        tf = 2 * M * N * K / (ms * 1e-3) / 1e12
        res[f"N{N}"] = {"us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1),
                        "mfma_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4), **quantiles_us(ts)}
        # A practical roof at the same shape: the vendor library's fp16 GEMM
        # (torch.matmul, hipBLASLt) over plain fp16 weights, so no dequantization
        # and an fp16 output. Measurement only; nothing in the library uses it.
        Wf = (torch.rand((K, N), generator=torch.Generator(device=dev).manual_seed(seed),
                         device=dev) - 0.5).to(torch.float16).contiguous()
        Yf = torch.empty((M, N), dtype=torch.float16, device=dev)
        for _ in range(warmup):
            torch.matmul(X, Wf, out=Yf)
        gv = capture(torch, lambda: [torch.matmul(X, Wf, out=Yf) for _ in range(4)])
        tv, _ = time_graph_dist(torch, [gv], max(steps, 64) // 4 + 1, 4)
        tfv = 2 * M * N * K / tv / 1e12
        res[f"N{N}"]["vendor_f16_gemm"] = {"us": round(tv * 1e6, 1), "TFLOPs": round(tfv, 1)}
        res[f"N{N}"]["frac_of_vendor"] = round(tf / tfv, 4)
        log(f"[prefill] N={N} vendor fp16 GEMM: {res[f'N{N}']['vendor_f16_gemm']}")
        del gv, Wf, Yf
    return res


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)

    if args.only == "traffic-probe":
        traffic_probe(torch, dev)
        return
    if args.only == "moe":
        print(json.dumps({"moe": bench_moe(torch, dev, args.steps, args.warmup)}), flush=True)
        return
    if args.only == "prefill":
        print(json.dumps({"prefill": bench_prefill(torch, dev, args.steps, args.warmup)}), flush=True)
        return
    if args.only == "probes":
        print(json.dumps({"probes": bench_probes(torch, dev)}), flush=True)
        return

    probes = bench_probes(torch, dev)
    d = bench_dense(torch, dev, args.steps, args.warmup)
    value = d["step_bytes"] / d["step_s"] / 1e9
    log(f"[dense] step {d['step_s'] * 1e3:.3f} ms (wall {d['wall_s'] * 1e3:.3f} ms), {value:.1f} GB/s")
    for k, v in d["per_call"].items():
        log(f"  {k:22s} {v}")
    roof = dense_roofline(d, probes)
    for k, v in d["per_call"].items():
        v["attainable_GBps"] = attainable_for(probes, v["bytes"])
        v["attainable_frac"] = round(v["GBps"] / v["attainable_GBps"], 4)
    extras = {"probes": probes}
    if not args.no_extras and args.only is None:
        extras["moe_decode"] = bench_moe(torch, dev, args.steps, args.warmup)
        extras["prefill_gemm"] = bench_prefill(torch, dev, args.steps, args.warmup)
        extras["q8_0_gemv"] = bench_q8(torch, dev, args.steps, args.warmup, d)
    extras["dense_per_call"] = d["per_call"]
    extras["dense_per_batch_GBps"] = {str(M): round(b / (ms * 1e-3) / 1e9, 1)
                                      for M, (ms, b) in d["per_M"].items()}
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        log("[cpu] timing the oracle")
        cpu = cpu_baselines(d, args.cpu_seconds)
    line = {
        "metric": "Q4_0 decode GEMV achieved HBM GB/s (dense 7B decode linears)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["step_s"] * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "dense 7B-shaped decode linears: Q4_0 4096x4096, 4096x11008 (x2), "
                               "11008x4096 at batch 1, 4 and 8 (12 GEMVs per step)",
                   "weights": "Q4_0 (18 B per 32 weights)", "rotation_copies": d["R"],
                   "hbm_frac": round(value / HBM_PEAK_GBS, 4),
                   "step_time": d["step_dist"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "also": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
