"""Throughput of the W4A16 linear layer on one MI355X.

Step: one decoder layer's four projections at M = 1 (qkv 2048->2560,
o 2048->2048, gate_up 2048->32768, down 16384->2048; bf16 activations,
weights N(0,0.02) with 1% N(0,0.2) outliers, RTN INT4 with group 128),
the decode workload the M = 1 HBM metric is quoted on.  The layer's weights
rotate over a pool of distinct copies (>= 1 GiB, more than the 256 MB
Infinity Cache plus L2) so every step streams its weights from HBM, as a
model with many layers would.  Inputs are resident in HBM before timing.

Timing: a timed region is exactly --steps steps between two device
synchronisations (HIP events on the replay stream); regions repeat until at
least 20 ms and 200 kernel launches have been timed, and ms_per_step is the
median over the regions.

value  = algorithmic bytes of the step (packed codes + FP32 scales + x + y)
         / measured time, in GB/s.
Also reported (same JSON line):
  roofline      the dominant kernel (gate_up, M = 1) against 8 TB/s: its
                average launch duration from HIP events (live), next to the
                mean of the committed rocprofv3 kernel trace of this command;
  m1024         the prefill projections at M = 1024 (fp16, bias) in TFLOP/s
                against the dense 2.5 PFLOP/s fp16 MFMA peak, with the oracle
                timed on a row sample of the same projections;
  m4096, c5_m1024  the roofline-sweep projections at M = 4096 and M = 1024
                (bf16) in TFLOP/s;
  load          quantize and pack kernel throughput (events, preallocated
                outputs), shard and in-place update rates;
  cpu_baseline  the CPU oracle on a bounded sample of the same step.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
    python bench.py --sweep [--sweep-out FILE]     # the 36-case table
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16/fp16
POOL_BYTES = 1 << 30
MIN_TIMED_MS = 20.0        # every timed figure covers at least this much GPU time
MIN_LAUNCHES = 200         # and at least this many kernel launches
CSRC = os.path.join(ROOT, "weight_only_int4_rtn_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_cases():
    import synth
    return [synth.case_by_name(n) for n in
            ("c3_qkv_m1_k2048_n2560", "c3_o_m1_k2048_n2048",
             "c3_gate_up_m1_k2048_n32768", "c3_down_m1_k16384_n2048")]


def prefill_cases():
    import synth
    return [c for c in synth.all_cases() if c.config == 4]


def sweep_cases_at(m):
    import synth
    return [c for c in synth.all_cases() if c.config == 5 and c.m == m]


def alg_bytes(c, bits=4):
    """Algorithmic HBM bytes of one projection: packed codes + FP32 scales +
    x + y (+ bias), each read or written once."""
    if bits == 4:
        return c.alg_bytes()
    return c.n * c.k + c.n * (c.k // 128) * 4 + 2 * c.m * c.k + 2 * c.m * c.n + (2 * c.n if c.bias else 0)


def floor_us(c, bits=4):
    """Time of one projection at 100 % of its bounding roofline."""
    return max(alg_bytes(c, bits) / (HBM_PEAK_GBS * 1e3), c.flops() / (MFMA_PEAK_TFLOPS * 1e6))


def sources_hash() -> str:
    """SHA-256 over the HIP library's sources: a committed profile taken on
    other sources no longer describes the kernels."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# pools, graphs, timing


def build_pool(cases, dev, bits=4):
    """Quantize + pack each case's weight once (INT4, or INT8 for bits=8),
    then copy it until the pool of layers exceeds POOL_BYTES.  Returns the
    layers (lists of packed weights, one per case)."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    packed0 = []
    for c in cases:
        w = synth.make_weight(c).to(dev)
        if bits == 8:
            codes, scales = w4.quantize_int8(w)
            p = w4.pack_int8(codes, scales)
        else:
            codes, scales = w4.quantize(w)
            p = w4.pack(codes, scales)
        packed0.append(p)
        del w, codes, scales
    per_layer = sum(p.numel() for p in packed0)
    copies = max(2, -(-POOL_BYTES // per_layer))
    layers = [packed0] + [[p.clone() for p in packed0] for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return layers


def capture(fn):
    """A HIP graph of fn() (torch.cuda.graph over the current device)."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def make_step(cases, layer, xs, biases, ys, workspace, bits=4):
    import weight_only_int4_rtn_amd as w4

    def step():
        for j, c in enumerate(cases):
            w4.linear(xs[j], layer[j], c.n, biases[j], out=ys[j], workspace=workspace, bits=bits)
    return step


def steps_per_graph(steps: int) -> int:
    """Consecutive steps (layers) per captured graph: the largest divisor of
    `steps` up to 16, so a timed region replays whole graphs."""
    return max(d for d in range(1, 17) if steps % d == 0)


def time_regions(graphs, per_graph, steps, warmup, launches_per_step):
    """Replay graphs of `per_graph` consecutive steps round-robin.  After the
    warmup, a timed region is exactly `steps` steps between two device
    synchronisations (HIP events on the replay stream); regions repeat until
    MIN_TIMED_MS and MIN_LAUNCHES are reached (at least three).  Returns
    (median ms per step, regions, total timed ms)."""
    import torch
    nxt = 0
    for _ in range(-(-warmup // per_graph)):
        graphs[nxt % len(graphs)].replay()
        nxt += 1
    stream = torch.cuda.current_stream()
    per_step, total_ms, launches = [], 0.0, 0
    while len(per_step) < 3 or total_ms < MIN_TIMED_MS or launches < MIN_LAUNCHES:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps // per_graph):
            graphs[nxt % len(graphs)].replay()
            nxt += 1
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        per_step.append(ms / steps)
        total_ms += ms
        launches += steps * launches_per_step
    return statistics.median(per_step), len(per_step), total_ms


def time_launch_graphs(graphs, launches_per_graph):
    """Median duration of one launch: each replay of a graph of back-to-back
    launches is timed with HIP events on its stream; replays (round-robin)
    repeat until MIN_TIMED_MS and MIN_LAUNCHES are reached (at least five).
    Returns (median us per launch, launches timed)."""
    import torch
    stream = torch.cuda.current_stream()
    for g in graphs[:2]:
        g.replay()
    per, total_ms, n, i = [], 0.0, 0, 0
    while len(per) < 5 or total_ms < MIN_TIMED_MS or n < MIN_LAUNCHES:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graphs[i % len(graphs)].replay()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        per.append(ms * 1e3 / launches_per_graph)
        total_ms += ms
        n += launches_per_graph
        i += 1
    return statistics.median(per), n


def time_kernel(case, layers, j, x, bias, y, workspace, launches=24, bits=4):
    """Median duration of one projection's launch, from HIP events on its
    stream around replays of a graph of back-to-back launches (weights rotate
    over distinct copies)."""
    import weight_only_int4_rtn_amd as w4

    def many():
        for i in range(launches):
            w4.linear(x, layers[i % len(layers)][j], case.n, bias, out=y, workspace=workspace, bits=bits)
    g = capture(many)
    us, _ = time_launch_graphs([g], launches)
    return us * 1e-3


def eager_ms(cases, layers, xs, biases, ys, workspace, steps=20):
    import torch
    for i in range(3):
        make_step(cases, layers[i % len(layers)], xs, biases, ys, workspace)()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        make_step(cases, layers[i % len(layers)], xs, biases, ys, workspace)()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def run_workload(cases, dev, steps, warmup, dominant, bits=4, eager=True, per_kernel=False):
    """Pool, graphs, timings for one workload.  Returns a dict of figures."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    layers = build_pool(cases, dev, bits)
    xs = [synth.make_x(c).to(dev) for c in cases]
    biases = [synth.make_bias(c).to(dev) if c.bias else None for c in cases]
    ys = [torch.empty((c.m, c.n), dtype=c.torch_dtype, device=dev) for c in cases]
    ws_bytes = max(w4.workspace_bytes(c.m, c.n, c.k, bits=bits) for c in cases)
    workspace = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    log(f"pool: {len(layers)} layers of {sum(p.numel() for p in layers[0]) / 1e6:.1f} MB; "
        f"paths {[w4.choose_path(c.m, c.n, c.k, bits).name for c in cases]}")
    # Each graph runs `per` consecutive layers of the pool, as a decode loop
    # runs a model's layers back to back; the graphs together cover the pool.
    per = steps_per_graph(steps)

    def layer_run(first):
        fns = [make_step(cases, layers[(first + i) % len(layers)], xs, biases, ys, workspace, bits)
               for i in range(per)]

        def run():
            for f in fns:
                f()
        return run
    graphs = [capture(layer_run(first)) for first in range(0, len(layers), per)]
    ms, regions, timed_ms = time_regions(graphs, per, steps, warmup, len(cases))
    kernel_ms = []
    for j, c in enumerate(cases):
        if per_kernel or j == dominant:
            kernel_ms.append(time_kernel(c, layers, j, xs[j], biases[j], ys[j], workspace, bits=bits))
        else:
            kernel_ms.append(None)
    eager = eager_ms(cases, layers, xs, biases, ys, workspace) if eager else None
    out = {"ms": ms, "dom_ms": kernel_ms[dominant], "kernel_ms": kernel_ms, "eager_ms": eager,
           "steps_per_graph": per, "regions": regions, "timed_ms": timed_ms}
    del graphs, layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# committed kernel-trace summaries (rocprofv3 --kernel-trace --stats)

TRACE_M1 = os.path.join(ROOT, "profiles", "gemv_m1_decode_layer_kernel_trace.md")
TRACE_M1024 = os.path.join(ROOT, "profiles", "gemm_m1024_prefill_kernel_trace.md")


def trace_kernel(c, bits=4):
    """(name pattern, grid in threads) that identify the kernel a case's
    automatic plan launches (its main kernel) in a kernel-trace summary."""
    import weight_only_int4_rtn_amd as w4
    e = w4.explain(c.m, c.n, c.k, bits=bits)
    act = 1 if c.dtype == "bf16" else 2
    grid = e["workgroups"] * e["waves"] * 64
    if e["path"] == w4.Path.GEMV:
        return rf"void w4a16::gemv_kernel<{min(c.m, 4)}, {act}, {e['waves']}, \d+, 0, {bits}>", grid
    if e["path"] == w4.Path.MGEMV:
        return rf"void w4a16::mgemv_kernel<\d+, {act}, {e['waves']}, \d+, 0, {bits}>", grid
    if e["path"] == w4.Path.SKINNY:
        # staged x (skinny_kernel) or x whole in LDS (skinny_direct_kernel)
        return (rf"void w4a16::skinny_(kernel<\d+, {act}, 0, \d+, {bits}>|direct_kernel<\d+, {act}, \d+, {bits}>)",
                grid)
    if e["waves"] == 8:
        sk = "true" if e["stream_k"] else "false"
        return rf"void w4a16::gemm8_kernel<{act}, (true|false), {bits}, {e['tile_m']}, {e['tile_n']}, {sk}>", grid
    return rf"void w4a16::gemm_kernel<{act}, 4>", grid


def trace_row(path, kernel, grid):
    """(mean us, launches, sources current?) of a kernel (name pattern, grid)
    in a committed trace summary, or None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    current = f"- sources_sha256: `{sources_hash()}`" in text
    for ln in text.splitlines():
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 6 and re.match(kernel, cells[0].strip("`")) and cells[1] == str(grid):
            try:
                return float(cells[3]), int(cells[2]), current
            except ValueError:
                return None
    return None


def trace_view(path, kernel, grid, live_us, work, peak, per_us):
    """The trace's figure for the dominant kernel beside the live one."""
    row = trace_row(path, kernel, grid)
    if row is None:
        return None
    mean_us, launches, current = row
    achieved = work / mean_us * per_us
    return {"file": os.path.relpath(path, ROOT), "kernel": kernel, "grid": grid, "launches": launches,
            "avg_launch_us": mean_us, "achieved": round(achieved, 2), "frac": round(achieved / peak, 4),
            "rel_diff_vs_live": round(mean_us / live_us - 1.0, 4), "sources_current": current}


# ---------------------------------------------------------------------------
# extra workloads


def ffn_block(act, m, hidden, inter, dtype, dev):
    """An FFN block (up or [up | gate] projection, then the down projection
    with the activation fused into its input) against the same block with
    the activation as separate torch kernels between two plain projections.
    Weights rotate over a >= 1 GiB pool; each variant is a HIP graph of 8
    consecutive blocks, timed with HIP events.  Returns us per block for both
    and the fused block's algorithmic GB/s."""
    import torch

    import weight_only_int4_rtn_amd as w4
    g = torch.Generator().manual_seed(1234)
    width = 2 * inter if act == w4.Act.SWIGLU else inter
    packs = []
    for n, k in ((width, hidden), (hidden, inter)):
        w = (torch.randn(n, k, generator=g) * 0.02).to(dev)
        c, sc = w4.quantize(w)
        packs.append(w4.pack(c, sc))
        del w, c, sc
    per = sum(p.numel() for p in packs)
    copies = max(2, -(-POOL_BYTES // per))
    pool = [packs] + [[p.clone() for p in packs] for _ in range(copies - 1)]
    x = torch.randn(m, hidden, generator=g).to(dtype).to(dev)
    bias = (torch.randn(hidden, generator=g) * 0.01).to(dtype).to(dev)
    u = torch.empty(m, width, dtype=dtype, device=dev)
    a = torch.empty(m, inter, dtype=dtype, device=dev)
    y = torch.empty(m, hidden, dtype=dtype, device=dev)
    ws = torch.zeros(max(16, w4.workspace_bytes(m, width, hidden), w4.workspace_bytes(m, hidden, inter, act)),
                     dtype=torch.uint8, device=dev)

    def fused(layer):
        w4.linear(x, layer[0], width, out=u, workspace=ws)
        w4.linear(u, layer[1], hidden, bias, out=y, workspace=ws, act=act)

    def unfused(layer):
        w4.linear(x, layer[0], width, out=u, workspace=ws)
        if act == w4.Act.SWIGLU:
            torch.mul(u[:, :inter], torch.nn.functional.silu(u[:, inter:]), out=a)
        else:
            a.copy_(torch.nn.functional.gelu(u, approximate="tanh"))
        w4.linear(a, layer[1], hidden, bias, out=y, workspace=ws)

    def timed(fn):
        per_graph = 8
        graphs = [capture(lambda f=first: [fn(pool[(f + i) % len(pool)]) for i in range(per_graph)])
                  for first in range(0, len(pool), per_graph)]
        us, _ = time_launch_graphs(graphs, per_graph)
        return us
    us_fused = timed(fused)
    us_unfused = timed(unfused)
    alg = (width * hidden + hidden * inter) * (0.5 + 4 / 128) + 2 * m * (hidden + width + width + hidden) + 2 * hidden
    del pool, packs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"us_fused": round(us_fused, 3), "us_unfused_torch_activation": round(us_unfused, 3),
            "fused_GBps": round(alg / (us_fused * 1e-6) / 1e9, 1)}


def events_us(fn, reps):
    """Mean us of fn() over `reps` eager calls, HIP events on the current stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def load_kernels(dev, reps=20):
    """Load-time rows a1-a3 on the decode layer's largest weight (gate_up,
    32768 x 2048 FP32): the quantize and pack kernels (and their INT8
    twins) timed with HIP events over preallocated outputs, so no
    allocation or host work is inside the timed region.  Bytes: quantize
    reads 4 B per weight and writes its codes and FP32 scales; pack reads
    those and writes the packed weight."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    c = synth.case_by_name("c3_gate_up_m1_k2048_n32768")
    n, k = c.n, c.k
    w = synth.make_weight(c).to(dev)
    codes = torch.empty(n, k // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(n, k // 128, dtype=torch.float32, device=dev)
    packed = torch.empty(w4.packed_bytes(n, k), dtype=torch.uint8, device=dev)
    q_us = events_us(lambda: w4.quantize(w, codes, scales), reps)
    p_us = events_us(lambda: w4.pack(codes, scales, out=packed), reps)
    sbytes = n * (k // 128) * 4
    q_bytes = n * k * 4 + n * k // 2 + sbytes
    p_bytes = n * k // 2 + sbytes + packed.numel()
    codes8, scales8 = w4.quantize_int8(w)
    q8_us = events_us(lambda: w4.quantize_int8(w), reps)
    p8_us = events_us(lambda: w4.pack_int8(codes8, scales8), reps)
    q8_bytes = n * k * 4 + n * k + sbytes
    p8_bytes = n * k + sbytes + w4.packed_bytes(n, k, 8)
    del w, codes, scales, packed, codes8, scales8
    torch.cuda.synchronize()

    def row(us, b):
        return {"us": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1),
                "pct_hbm_peak": round(100 * b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1), "bytes": b}
    return {"workload": "gate_up weight 32768x2048 fp32, load time",
            "quantize": row(q_us, q_bytes), "pack": row(p_us, p_bytes),
            "quantize_int8": {**row(q8_us, q8_bytes), "note": "includes its output allocation"},
            "pack_int8": {**row(p8_us, p8_bytes), "note": "includes its output allocation"}}


def update_rate(dev, rank=16, replays=5):
    """A seeded low-rank merge (LoRA, rank 16) into the decode layer's gate_up
    weight, requantized in place with stochastic rounding: microseconds and
    the packed weight's bytes read + written per second."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    c = synth.case_by_name("c3_gate_up_m1_k2048_n32768")
    codes, scales = w4.quantize(synth.make_weight(c).to(dev))
    packed = w4.pack(codes, scales)
    del codes, scales
    g = torch.Generator().manual_seed(7)
    m1 = (torch.randn(c.n, rank, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    m2 = (torch.randn(rank, c.k, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    w4.update_(packed, c.n, c.k, mat1=m1, mat2=m2, alpha=0.5, seed=1)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(replays):
        w4.update_(packed, c.n, c.k, mat1=m1, mat2=m2, alpha=0.5, seed=2 + i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / replays
    return {"workload": f"rank-{rank} bf16 merge into gate_up 32768x2048, stochastic rounding",
            "us": round(us, 2), "packed_GBps": round(2 * packed.numel() / (us * 1e-6) / 1e9, 1)}


def shard_rate(dev, parts=8, replays=5):
    """Tensor-parallel shards of the decode layer's gate_up (rows, dim 0) and
    down (group-aligned columns, dim 1) weights, `parts` each, from packed
    weights without requantizing: bytes read + written per second."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    work = []
    for name, dim in (("c3_gate_up_m1_k2048_n32768", 0), ("c3_down_m1_k16384_n2048", 1)):
        c = synth.case_by_name(name)
        codes, scales = w4.quantize(synth.make_weight(c).to(dev))
        work.append((w4.pack(codes, scales), c.n, c.k, dim))
        del codes, scales

    def run():
        outs = []
        for packed, n, k, dim in work:
            size = (n if dim == 0 else k) // parts
            outs += [w4.shard(packed, n, k, dim, i * size, size) for i in range(parts)]
        return outs
    run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        outs = run()
    e1.record(stream)
    torch.cuda.synchronize()
    moved = 2 * sum(o.numel() for o in outs)
    return round(moved * replays / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel: two rocprofv3 counter runs of
# `bench.py --traffic-probe` (FETCH_SIZE, then WRITE_SIZE), scaled by what the
# same counters read for an elementwise kernel of known size.  The summary
# records a hash of the kernel's sources; a changed kernel reports null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_gate_up_m1_traffic.md")
TRAFFIC_SOURCES = [os.path.join(CSRC, f) for f in ("gemv.hip", "common.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the gate_up GEMV from the committed counter
    summary, or None when it is missing or was taken on other sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            fields = dict(ln.split(":", 1) for ln in fh.read().splitlines() if ln.startswith("- ") and ":" in ln)
    except OSError:
        return None
    fields = {k[2:].strip(): v.strip().strip("`") for k, v in fields.items()}
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_probe(dev):
    """Launches for the counter runs: the gate_up GEMV on 16 pool copies, then
    an elementwise kernel over 256 MiB (reads and writes exactly that much),
    the scale for the counters."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    c = synth.case_by_name("c3_gate_up_m1_k2048_n32768")
    layers = build_pool([c], dev)
    x = synth.make_x(c).to(dev)
    y = torch.empty((c.m, c.n), dtype=c.torch_dtype, device=dev)
    for i in range(16):
        w4.linear(x, layers[i % len(layers)][0], c.n, out=y)
    torch.cuda.synchronize()
    src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"traffic probe: 16 GEMV launches ({c.alg_bytes()} algorithmic bytes each), "
        f"4 elementwise launches of {src.numel() * 4} bytes read + written; sources {kernel_source_hash()}")


def probe(dev, names, launches=8):
    """Launches for counter runs: each named case `launches` times eagerly
    over distinct weight copies (the first dispatch of each is dropped by the
    summaries)."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    for name in names:
        c = synth.case_by_name(name)
        layers = build_pool([c], dev)
        x = synth.make_x(c).to(dev)
        bias = synth.make_bias(c).to(dev) if c.bias else None
        y = torch.empty((c.m, c.n), dtype=c.torch_dtype, device=dev)
        ws = torch.zeros(max(w4.workspace_bytes(c.m, c.n, c.k), 16), dtype=torch.uint8, device=dev)
        for i in range(launches):
            w4.linear(x, layers[i % len(layers)][0], c.n, bias, out=y, workspace=ws)
        torch.cuda.synchronize()
        log(f"probe: {launches} launches of {c.name} on the {w4.choose_path(c.m, c.n, c.k).name} path")
        del layers
        torch.cuda.empty_cache()


GEMM_PROBE_CASE = "c4_m1024_k2048_n32768"

# SQ counters in two rocprofv3 --pmc passes (at most 8 SQ counters a pass):
# SQ_*_CYCLES wave counters count quad-cycles (4 clocks); the MFMA busy
# counter counts clocks summed over the 1024 SIMDs.
SQ_PASSES = (
    ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
     "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"),
    ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
     "SQ_ACTIVE_INST_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"),
)


def summarize_sq(dbs, match="gemm"):
    """Markdown summary of the SQ counters of the kernels whose name contains
    `match`, from counter databases of a probe run: mean per dispatch (first
    dispatch dropped), per-wave counts, and the shares of a wave's lifetime
    spent issuing, waiting on its counters or a barrier, and waiting to
    issue."""
    vals = {}
    name = None
    for db in dbs:
        rows = _rocpd_rows(db, "select dispatch_id, kernel_name, counter_name, value from counters_collection")
        per = {}
        for d, kname, cname, v in rows:
            if match not in kname:
                continue
            name = kname.split("(")[0]
            per.setdefault(cname, {}).setdefault(d, 0.0)
            per[cname][d] += v
        for cname, byd in per.items():
            v = [byd[d] for d in sorted(byd)]
            v = v[1:] if len(v) > 1 else v
            vals[cname] = sum(v) / len(v)
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {match!r} in the counter databases")
    lines = [f"Kernel `{name}`; mean per dispatch:", "", "| counter | value |", "|---|---:|"]
    lines += [f"| {k} | {vals[k]:,.0f} |" for k in sorted(vals)]
    waves = vals.get("SQ_WAVES")
    if waves:
        lines += ["", "Per wave:"]
        for k, what in (("SQ_INSTS_MFMA", "MFMA instructions"), ("SQ_INSTS_VALU", "VALU instructions (MFMA included)"),
                        ("SQ_INSTS_LDS", "LDS instructions"), ("SQ_INSTS_VMEM", "vector memory instructions"),
                        ("SQ_INSTS_SALU", "scalar ALU instructions")):
            if k in vals:
                lines.append(f"- {what}: {vals[k] / waves:,.1f}")
    life = vals.get("SQ_WAVE_CYCLES")
    if life:
        lines += ["", "Share of the waves' lifetime (quad-cycles over SQ_WAVE_CYCLES):"]
        for k, what in (("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_WAIT_ANY", "waiting on s_waitcnt or a barrier"),
                        ("SQ_WAIT_INST_ANY", "ready but waiting to issue (dependency or a busy unit)"),
                        ("SQ_WAIT_INST_LDS", "waiting to issue an LDS instruction")):
            if k in vals:
                lines.append(f"- {what}: {100 * vals[k] / life:.1f} %")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
        lines += ["", f"MFMA busy clocks per SIMD (over 1024 SIMDs): {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024:,.0f}"]
    return "\n".join(lines)


def _rocpd_rows(db, sql):
    import sqlite3
    con = sqlite3.connect(db)
    try:
        return con.execute(sql).fetchall()
    finally:
        con.close()


def summarize_trace(db):
    """Markdown table of a rocprofv3 --kernel-trace database: launches and
    durations per kernel name and grid size (the `kernels` view)."""
    rows = _rocpd_rows(db, "select name, grid_x, duration from kernels")
    groups = {}
    for name, grid, dur in rows:
        groups.setdefault((name, grid), []).append(dur / 1e3)
    lines = ["| kernel | grid (threads) | launches | mean us | median us | min us |",
             "|---|---:|---:|---:|---:|---:|"]
    for (name, grid), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        short = name.split("(")[0]
        lines.append(f"| `{short}` | {grid} | {len(d)} | {statistics.mean(d):.2f} | "
                     f"{statistics.median(d):.2f} | {min(d):.2f} |")
    return "\n".join(lines)


def summarize_traffic(fetch_db, write_db):
    """HBM bytes per launch of the gate_up GEMV from two counter databases of
    `bench.py --traffic-probe` (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by what its counter reads for the elementwise
    kernel that reads and writes exactly 256 MiB."""
    known_kib = (64 << 20) * 4 / 1024

    def per_dispatch(db, counter):
        rows = _rocpd_rows(db, "select dispatch_id, kernel_name, grid_size, value from counters_collection "
                               f"where counter_name = '{counter}'")
        acc = {}
        for d, name, grid, v in rows:
            key = (d, name, grid)
            acc[key] = acc.get(key, 0.0) + v
        return acc

    out = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        acc = per_dispatch(db, counter)
        gemv = [v for (d, name, g), v in acc.items() if "gemv_kernel" in name]
        copy = [v for (d, name, g), v in acc.items()
                if "elementwise" in name and g == (64 << 20) // 4 and v > known_kib / 8]
        if not gemv or not copy:
            raise SystemExit(f"{db}: no GEMV or no 256 MiB elementwise dispatch with {counter}")
        scale = known_kib / (sum(copy) / len(copy))
        out[counter] = (sum(gemv) / len(gemv), scale, len(gemv), len(copy))
    fetch = out["FETCH_SIZE"][0] * out["FETCH_SIZE"][1] * 1024
    write = out["WRITE_SIZE"][0] * out["WRITE_SIZE"][1] * 1024
    return out, int(round(fetch + write))


# ---------------------------------------------------------------------------
# CPU oracle baselines (test infrastructure, timed here as a reported baseline)


def cpu_baseline(cases, target_seconds=10.0):
    """The oracle (as it stands) on the same M = 1 decode layer, repeated."""
    import oracle
    import synth
    prepared = []
    for c in cases:
        q, s = oracle.quantize(synth.make_weight(c).numpy())
        xb = synth.to_bits16(synth.make_x(c))
        prepared.append((c, xb, q, s))
    bytes_per_pass = sum(c.alg_bytes() for c in cases)
    reps = 0
    t0 = time.perf_counter()
    while True:
        for c, xb, q, s in prepared:
            oracle.linear(xb, oracle.BF16, q, s)
        reps += 1
        if time.perf_counter() - t0 >= target_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": round(bytes_per_pass * reps / el / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the full M=1 decode layer (4 projections, {bytes_per_pass / 1e6:.1f} MB of "
                      f"algorithmic bytes) run {reps} times in {el:.1f} s",
            "ms_per_step": round(el * 1e3 / reps, 2)}


def oracle_rows_time(c, rows, q=None, s=None):
    """Seconds the oracle's linear takes on the first `rows` rows of the
    case's x (quantizing the weight first if q, s are not given)."""
    import oracle
    import synth
    if q is None:
        q, s = oracle.quantize(synth.make_weight(c).numpy())
    xb = synth.to_bits16(synth.make_x(c))[:rows]
    bb = synth.to_bits16(synth.make_bias(c)) if c.bias else None
    t0 = time.perf_counter()
    oracle.linear(xb, oracle.BF16 if c.dtype == "bf16" else oracle.F16, q, s, bb)
    return time.perf_counter() - t0


def cpu_baseline_rows(cases, target_seconds=8.0):
    """The oracle on a row sample of large-M projections: each projection's
    first `rows` rows of x against its whole weight, the row count doubled
    from 4 until one pass takes `target_seconds` (or all rows); TFLOP/s over
    the sample (the oracle's cost is linear in the rows)."""
    import oracle
    import synth
    prepared = [(c, *oracle.quantize(synth.make_weight(c).numpy())) for c in cases]
    rows = 4
    while True:
        total_s, flops = 0.0, 0
        for c, q, s in prepared:
            total_s += oracle_rows_time(c, rows, q, s)
            flops += 2 * rows * c.n * c.k
        if total_s >= target_seconds or rows >= cases[0].m:
            break
        rows = min(cases[0].m, rows * max(2, int(target_seconds / max(total_s, 1e-3) * 0.6)))
    return {"value": round(flops / total_s / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the first {rows} of {cases[0].m} rows of each of the {len(cases)} projections "
                      f"({flops / 1e9:.2f} GFLOP) in {total_s:.1f} s",
            "extrapolated_ms_per_step": round(total_s * cases[0].m / rows * 1e3, 1)}


# ---------------------------------------------------------------------------
# the 36-case table


def sweep(dev, out_path=None, with_oracle=True, only=None, oracle_gflop=2.0):
    """Every case of the five workloads: per-launch GPU time (HIP events,
    graphs of back-to-back launches rotating over >= 1 GiB of distinct
    (packed weight, x, y) sets, >= 20 ms and >= 200 launches, median over
    replays), GB/s, TFLOP/s, the fraction of each roofline, the kernel path,
    and the oracle's time (quantize on the whole weight; linear on a row
    sample of at most `oracle_gflop` GFLOP, scaled to all rows)."""
    import torch

    import oracle
    import synth
    import weight_only_int4_rtn_amd as w4
    rows = []
    for c in synth.all_cases():
        if only and not any(s in c.name for s in only):
            continue
        w_cpu = synth.make_weight(c)
        codes, scales = w4.quantize(w_cpu.to(dev))
        p = w4.pack(codes, scales)
        del codes, scales
        x = synth.make_x(c).to(dev)
        bias = synth.make_bias(c).to(dev) if c.bias else None
        per_set = p.numel() + x.numel() * 2 + c.m * c.n * 2
        sets = max(2, -(-POOL_BYTES // per_set))
        packs = [p] + [p.clone() for _ in range(sets - 1)]
        xs = [x] + [x.clone() for _ in range(sets - 1)]
        ys = [torch.empty((c.m, c.n), dtype=c.torch_dtype, device=dev) for _ in range(sets)]
        ws = torch.zeros(max(w4.workspace_bytes(c.m, c.n, c.k), 16), dtype=torch.uint8, device=dev)
        per_graph = min(sets, 64)

        def run(first):
            for i in range(per_graph):
                j = (first + i) % sets
                w4.linear(xs[j], packs[j], c.n, bias, out=ys[j], workspace=ws)
        graphs = [capture(lambda f=first: run(f)) for first in range(0, sets, per_graph)]
        us, launches = time_launch_graphs(graphs, per_graph)
        del graphs, packs, xs, ys, ws, p, x
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        b, f = c.alg_bytes(), c.flops()
        gbs, tfs = b / (us * 1e-6) / 1e9, f / (us * 1e-6) / 1e12
        row = {"case": c.name, "config": c.config, "m": c.m, "k": c.k, "n": c.n, "dtype": c.dtype,
               "bias": c.bias, "path": w4.choose_path(c.m, c.n, c.k).name, "us": round(us, 3),
               "launches": launches, "GBps": round(gbs, 1), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 2),
               "TFLOPs": round(tfs, 2), "pct_mfma": round(100 * tfs / MFMA_PEAK_TFLOPS, 2),
               "bound": "hbm" if b / HBM_PEAK_GBS >= f / (MFMA_PEAK_TFLOPS * 1e3) else "mfma",
               "pct_roofline": round(100 * floor_us(c) / us, 2)}
        if with_oracle:
            t0 = time.perf_counter()
            q, s = oracle.quantize(w_cpu.numpy())
            row["oracle_quantize_s"] = round(time.perf_counter() - t0, 3)
            r = max(1, min(c.m, int(oracle_gflop * 1e9 // (2 * c.n * c.k))))
            t = oracle_rows_time(c, r, q, s)
            row["oracle_linear_s"] = round(t * c.m / r, 3)
            row["oracle_rows_timed"] = r
            row["oracle_cores"] = oracle.num_threads()
        rows.append(row)
        log(json.dumps(row))
        if out_path:
            with open(out_path, "a") as fh:
                fh.write(json.dumps(row) + "\n")
    return rows


def sweep_table(rows):
    """Markdown table of sweep rows."""
    hdr = ("| case | M | K | N | path | us | GB/s | %HBM | TFLOP/s | %MFMA | bound | %roofline | "
           "oracle linear s | oracle quant s |")
    lines = [hdr, "|---|---:|---:|---:|---|---:|---:|---:|---:|---:|---|---:|---:|---:|"]
    for r in rows:
        ol = r.get("oracle_linear_s")
        oq = r.get("oracle_quantize_s")
        note = "" if r.get("oracle_rows_timed", r["m"]) == r["m"] else f" ({r['oracle_rows_timed']} rows)"
        lines.append(f"| {r['case']} | {r['m']} | {r['k']} | {r['n']} | {r['path']} | {r['us']:.2f} | "
                     f"{r['GBps']:.0f} | {r['pct_hbm']:.1f} | {r['TFLOPs']:.1f} | {r['pct_mfma']:.1f} | "
                     f"{r['bound']} | {r['pct_roofline']:.1f} | "
                     f"{'' if ol is None else f'{ol:.3f}{note}'} | {'' if oq is None else f'{oq:.3f}'} |")
    return "\n".join(lines)


# ---------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the decode step, the M = 1024 / 4096 legs and the baselines")
    ap.add_argument("--sweep", action="store_true", help="time all 36 cases and print the table")
    ap.add_argument("--sweep-out", metavar="FILE", help="append one JSON line per sweep case to FILE")
    ap.add_argument("--sweep-only", nargs="+", metavar="SUBSTR", help="sweep only cases whose name contains one")
    ap.add_argument("--summarize-sweep", metavar="JSONL", help="print the table of a --sweep-out file and exit")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only the launches the HBM counter runs measure (see TRAFFIC_FILE)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only the launches the GEMM stall-counter runs measure (8 launches of the M = 1024 GEMM)")
    ap.add_argument("--probe", nargs="+", metavar="CASE", help="only 8 launches of each named case (counter runs)")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DB",
                    help="print the SQ counter summary of probe counter databases and exit")
    ap.add_argument("--sq-match", default="gemm", help="kernel-name substring for --summarize-sq")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace database and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write TRAFFIC_FILE from the two counter databases of --traffic-probe and exit")
    ap.add_argument("--sources-hash", action="store_true", help="print the hash of the HIP sources and exit")
    args = ap.parse_args()
    if args.sources_hash:
        print(sources_hash())
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        print(f"\n- sources_sha256: `{sources_hash()}`")
        return
    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq, args.sq_match))
        return
    if args.summarize_sweep:
        with open(args.summarize_sweep) as fh:
            print(sweep_table([json.loads(ln) for ln in fh if ln.strip()]))
        return
    if args.summarize_traffic:
        parts, traffic = summarize_traffic(*args.summarize_traffic)
        fk, fs, fn, fc = parts["FETCH_SIZE"]
        wk, wsc, wn, wc = parts["WRITE_SIZE"]
        text = "\n".join([
            "# HBM traffic of the gate_up GEMV at M = 1 (K 2048, N 32768, bf16)",
            "",
            "Commands (MI355X, one GPU; R = repository root, OUT = an output directory):",
            "",
            "    cd /tmp && export TMPDIR=/tmp",
            "    timeout -s KILL 60 rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_fetch -o run -- python3 $R/bench.py --traffic-probe",
            "    timeout -s KILL 60 rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_write -o run -- python3 $R/bench.py --traffic-probe",
            "    python3 $R/bench.py --summarize-traffic $OUT/pmc_fetch/run_results.db $OUT/pmc_write/run_results.db",
            "",
            "The probe launches the GEMV 16 times over distinct weight copies and an",
            "elementwise kernel that reads and writes exactly 256 MiB; each counter is",
            "scaled by what it reads for that kernel.",
            "",
            f"- FETCH_SIZE per GEMV launch (KiB, mean of {fn}): {fk:.2f}; scale {fs:.5f} (from {fc} copies)",
            f"- WRITE_SIZE per GEMV launch (KiB, mean of {wn}): {wk:.2f}; scale {wsc:.5f} (from {wc} copies)",
            "- algorithmic_bytes_per_launch: `35721216`",
            f"- traffic_bytes_per_launch: `{traffic}`",
            f"- traffic / algorithmic: {traffic / 35721216:.4f}",
            f"- kernel_source_sha256: `{kernel_source_hash()}`",
            ""])
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as fh:
            fh.write(text)
        print(text)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer runs on one MI355X per process, and "
              "sharding it across GPUs is described in the design notes, not implemented", file=sys.stderr)
        sys.exit(2)

    import torch

    import weight_only_int4_rtn_amd as w4
    dev = torch.device("cuda:0")
    w4.lib()
    if args.traffic_probe:
        traffic_probe(dev)
        return
    if args.gemm_probe:
        probe(dev, [GEMM_PROBE_CASE])
        return
    if args.probe:
        probe(dev, args.probe)
        return
    if args.sweep:
        rows = sweep(dev, args.sweep_out, not args.no_cpu_baseline, args.sweep_only)
        print(sweep_table(rows), flush=True)
        return

    # --- decode step (M = 1) --------------------------------------------------
    cases = decode_cases()
    dominant = 2  # gate_up: the largest stream
    log(f"decode workload: {[c.name for c in cases]}")
    dec = run_workload(cases, dev, args.steps, args.warmup, dominant, per_kernel=True)
    ms, dom_ms = dec["ms"], dec["dom_ms"]
    step_bytes = sum(c.alg_bytes() for c in cases)
    value = step_bytes / (ms * 1e-3) / 1e9
    dom = cases[dominant]
    dom_gbs = dom.alg_bytes() / (dom_ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.2f} us/step (graph replay, median of {dec['regions']} regions, "
        f"{dec['timed_ms']:.1f} ms timed), {value:.1f} GB/s; eager {dec['eager_ms'] * 1e3:.1f} us/step; "
        f"gate_up {dom_ms * 1e3:.2f} us/launch, {dom_gbs:.1f} GB/s")
    per_proj = {c.name: {"us": round(t * 1e3, 3), "GBps": round(c.alg_bytes() / (t * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100 * c.alg_bytes() / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
                for c, t in zip(cases, dec["kernel_ms"])}

    # --- prefill (M = 1024, fp16, bias) ----------------------------------------
    pcases = prefill_cases()
    pdom = 1  # N = 32768: the largest GEMM
    log(f"prefill workload: {[c.name for c in pcases]}")
    pre = run_workload(pcases, dev, args.prefill_steps, 5, pdom, eager=False, per_kernel=True)
    pms, pdom_ms = pre["ms"], pre["dom_ms"]
    pflops = sum(c.flops() for c in pcases)
    ptf = pflops / (pms * 1e-3) / 1e12
    pd = pcases[pdom]
    pd_tf = pd.flops() / (pdom_ms * 1e-3) / 1e12
    log(f"prefill: {pms * 1e3:.1f} us/step, {ptf:.1f} TFLOP/s; N=32768 {pdom_ms * 1e3:.1f} us, {pd_tf:.1f} TFLOP/s")

    def proj_table(cs, kms):
        return {c.name: {"us": round(t * 1e3, 2), "TFLOPs": round(c.flops() / (t * 1e-3) / 1e12, 1),
                         "pct_mfma_peak": round(100 * c.flops() / (t * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 2),
                         "path": w4.choose_path(c.m, c.n, c.k).name} for c, t in zip(cs, kms)}

    # --- roofline-sweep projections at M = 4096 and 1024 (bf16) -------------
    big = {}
    for m in (4096, 1024):
        cs = sweep_cases_at(m)
        log(f"c5 M={m} workload: {[c.name for c in cs]}")
        r = run_workload(cs, dev, 10, 2, 1, eager=False, per_kernel=True)
        fl = sum(c.flops() for c in cs)
        tf = fl / (r["ms"] * 1e-3) / 1e12
        big[m] = {"workload": f"roofline sweep M={m} bf16: K1024xN4096, K2048xN16384, K16384xN2048 "
                              "(x with every 64th feature x10, one zero group per row)",
                  "tflops": round(tf, 2), "ms_per_step": round(r["ms"], 4),
                  "pct_mfma_peak": round(100 * tf / MFMA_PEAK_TFLOPS, 2),
                  "projections": proj_table(cs, r["kernel_ms"])}
        log(f"c5 M={m}: {r['ms'] * 1e3:.1f} us/step, {tf:.1f} TFLOP/s")

    extras = {}
    if not args.no_extras:
        # --- FFN blocks with the activation fused into the down projection --
        log("ffn blocks")
        extras["ffn"] = {
            "swiglu_m1": {"workload": "M=1 bf16: [up | gate] 2048x32768, down 16384x2048 with up*silu(gate) fused",
                          **ffn_block(w4.Act.SWIGLU, 1, 2048, 16384, torch.bfloat16, dev)},
            "gelu_m50": {"workload": "M=50 bf16: up 1024x4096, down 4096x1024 (+bias) with tanh-GELU fused",
                         **ffn_block(w4.Act.GELU_TANH, 50, 1024, 4096, torch.bfloat16, dev)},
        }
        log(f"ffn: {extras['ffn']}")
        # --- the same decode step with INT8 weights (W8A16) ------------------
        log("w8a16 decode workload")
        w8 = run_workload(cases, dev, args.steps, args.warmup, dominant, bits=8, eager=False)
        w8_bytes = sum(alg_bytes(c, 8) for c in cases)
        w8_gbs = w8_bytes / (w8["ms"] * 1e-3) / 1e9
        w8_dom_gbs = alg_bytes(dom, 8) / (w8["dom_ms"] * 1e-3) / 1e9
        w8a16 = {"workload": "decode layer M=1 as above with int8 g128 weights (amax/127)",
                 "GBps": round(w8_gbs, 2), "ms_per_step": round(w8["ms"], 5), "bytes_per_step": w8_bytes,
                 "pct_hbm_peak": round(100 * w8_gbs / HBM_PEAK_GBS, 2),
                 "roofline": {"bound": "hbm", "achieved": round(w8_dom_gbs, 2), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(w8_dom_gbs / HBM_PEAK_GBS, 4),
                              "kernel": f"{w4.choose_path(1, dom.n, dom.k, 8).name} int8 {dom.name}",
                              "avg_launch_us": round(w8["dom_ms"] * 1e3, 3), "bytes_per_launch": alg_bytes(dom, 8)}}
        pre8 = run_workload(pcases, dev, args.prefill_steps, 3, pdom, bits=8, eager=False)
        p8tf = pflops / (pre8["ms"] * 1e-3) / 1e12
        p8d_tf = pd.flops() / (pre8["dom_ms"] * 1e-3) / 1e12
        w8a16["m1024"] = {"workload": "prefill M=1024 fp16 with bias as above, int8 g128 weights",
                          "tflops": round(p8tf, 2), "ms_per_step": round(pre8["ms"], 4),
                          "pct_mfma_peak": round(100 * p8tf / MFMA_PEAK_TFLOPS, 2),
                          "roofline": {"bound": "mfma", "achieved": round(p8d_tf, 2), "peak": MFMA_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(p8d_tf / MFMA_PEAK_TFLOPS, 4),
                                       "kernel": f"{w4.choose_path(pd.m, pd.n, pd.k, 8).name} int8 {pd.name}",
                                       "avg_launch_us": round(pre8["dom_ms"] * 1e3, 3)}}
        extras["w8a16"] = w8a16
        log(f"w8a16: {w8a16}")
        log("load-time kernels")
        extras["load"] = {"kernels": load_kernels(dev), "shard_GBps": shard_rate(dev), "update": update_rate(dev),
                          "shard": "8 row shards of gate_up 32768x2048 and 8 column shards of down 2048x16384, "
                                   "packed to packed, eager launches"}

    out = {
        "metric": "W4A16 GEMM: HBM GB/s & %peak at M=1; TFLOP/s & %MFMA peak at M=1024",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; weights rotate over a >=1 GiB pool of layer copies; "
                f"steps replayed as HIP graphs of {dec['steps_per_graph']} consecutive layers; "
                f"median of {dec['regions']} timed regions of {args.steps} steps, {dec['timed_ms']:.1f} ms timed)",
        "config": {"workload": "decode layer M=1: qkv 2048x2560, o 2048x2048, gate_up 2048x32768, "
                               "down 16384x2048; bf16 x, int4 g128 weights",
                   "m": 1, "bytes_per_step": step_bytes, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "kernel_path": w4.choose_path(1, 2048, 2048).name,
                   "eager_ms_per_step": round(dec["eager_ms"], 4), "projections": per_proj},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "kernel": f"{w4.choose_path(1, dom.n, dom.k).name} {dom.name}",
                     "avg_launch_us": round(dom_ms * 1e3, 3), "bytes_per_launch": dom.alg_bytes(),
                     "trace": trace_view(TRACE_M1, *trace_kernel(dom), dom_ms * 1e3, dom.alg_bytes(),
                                         HBM_PEAK_GBS, 1e-3)},
        "m1024": {"workload": "prefill M=1024 fp16 with bias: K2048xN2560, K2048xN32768, K16384xN2048",
                  "tflops": round(ptf, 2), "ms_per_step": round(pms, 4),
                  "pct_mfma_peak": round(100 * ptf / MFMA_PEAK_TFLOPS, 2),
                  "projections": proj_table(pcases, pre["kernel_ms"]),
                  "roofline": {"bound": "mfma", "achieved": round(pd_tf, 2), "peak": MFMA_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(pd_tf / MFMA_PEAK_TFLOPS, 4),
                               "kernel": f"{w4.choose_path(pd.m, pd.n, pd.k).name} {pd.name}",
                               "avg_launch_us": round(pdom_ms * 1e3, 3), "flops_per_launch": pd.flops(),
                               "trace": trace_view(TRACE_M1024, *trace_kernel(pd), pdom_ms * 1e3, pd.flops(),
                                                   MFMA_PEAK_TFLOPS, 1e-6)}},
        "m4096": big[4096],
        "c5_m1024": big[1024],
        **extras,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baselines")
        out["cpu_baseline"] = cpu_baseline(cases)
        out["m1024"]["cpu_baseline"] = cpu_baseline_rows(pcases)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
