"""Throughput of the W4A16 linear layer on one MI355X.

Step: one decoder layer's four projections at M = 1 (qkv 2048->2560,
o 2048->2048, gate_up 2048->32768, down 16384->2048; bf16 activations,
weights N(0,0.02) with 1% N(0,0.2) outliers, RTN INT4 with group 128),
the decode workload the M = 1 HBM metric is quoted on.  The layer's weights
rotate over a pool of distinct copies (>= 1 GiB, more than the 256 MB
Infinity Cache plus L2) so every step streams its weights from HBM, as a
model with many layers would.  Inputs are resident in HBM before timing.

value  = algorithmic bytes of the step (packed codes + FP32 scales + x + y)
         / measured time, in GB/s.
Also reported (same JSON line):
  roofline      the dominant kernel (gate_up, M = 1) against 8 TB/s, its
                average duration from HIP events on its stream;
  m1024         the prefill projections at M = 1024 (fp16, bias) in TFLOP/s
                against the dense 2.5 PFLOP/s fp16 MFMA peak;
  load          quantize + pack throughput (load-time rows of the path);
  cpu_baseline  the CPU oracle on a bounded sample of the same step.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16/fp16
POOL_BYTES = 1 << 30


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


def build_pool(cases, dev, bits=4):
    """Quantize + pack each case's weight once (INT4, or INT8 for bits=8),
    then copy it until the pool of layers exceeds POOL_BYTES.  Returns
    (layers, load_stats)."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    packed0 = []
    load_bytes = 0
    load_time = 0.0
    for c in cases:
        w = synth.make_weight(c).to(dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if bits == 8:
            codes, scales = w4.quantize_int8(w)
            p = w4.pack_int8(codes, scales)
        else:
            codes, scales = w4.quantize(w)
            p = w4.pack(codes, scales)
        torch.cuda.synchronize()
        load_time += time.perf_counter() - t0
        # quantize reads W (4 B) and writes codes + scales; pack reads those and writes packed
        load_bytes += c.n * c.k * 4 + 2 * (c.n * c.k * bits // 8 + c.n * (c.k // 128) * 4) + p.numel()
        packed0.append(p)
        del w, codes, scales
    per_layer = sum(p.numel() for p in packed0)
    copies = max(2, -(-POOL_BYTES // per_layer))
    layers = [packed0] + [[p.clone() for p in packed0] for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return layers, {"bytes": load_bytes, "seconds": load_time}


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
    `steps` up to 16, so the timed region replays whole graphs."""
    return max(d for d in range(1, 17) if steps % d == 0)


def time_graphs(graphs, per_graph, steps, warmup):
    """Replay graphs of `per_graph` consecutive steps round-robin: warmup,
    then exactly `steps` timed steps between two device synchronisations,
    measured with HIP events on the replay stream.  Returns ms per step."""
    import torch
    for i in range(-(-warmup // per_graph)):
        graphs[i % len(graphs)].replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps // per_graph):
        graphs[i % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_kernel(case, layers, j, x, bias, y, workspace, launches=24, replays=10, bits=4):
    """Average duration of one projection's launch, from HIP events on its
    stream around replays of a graph of back-to-back launches (weights rotate
    over distinct copies)."""
    import torch

    import weight_only_int4_rtn_amd as w4

    def many():
        for i in range(launches):
            w4.linear(x, layers[i % len(layers)][j], case.n, bias, out=y, workspace=workspace, bits=bits)
    g = capture(many)
    g.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / (launches * replays)


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


def alg_bytes(c, bits=4):
    """Algorithmic HBM bytes of one projection: packed codes + FP32 scales +
    x + y (+ bias), each read or written once."""
    if bits == 4:
        return c.alg_bytes()
    return c.n * c.k + c.n * (c.k // 128) * 4 + 2 * c.m * c.k + 2 * c.m * c.n + (2 * c.n if c.bias else 0)


def run_workload(cases, dev, steps, warmup, dominant, bits=4, eager=True):
    """Pool, graphs, timings for one workload.  Returns a dict of figures."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    layers, load = build_pool(cases, dev, bits)
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
    ms = time_graphs(graphs, per, steps, warmup)
    dom = cases[dominant]
    dom_ms = time_kernel(dom, layers, dominant, xs[dominant], biases[dominant], ys[dominant], workspace,
                         bits=bits)
    eager = eager_ms(cases, layers, xs, biases, ys, workspace) if eager else None
    out = {"ms": ms, "dom_ms": dom_ms, "eager_ms": eager, "load": load, "steps_per_graph": per}
    del graphs, layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def ffn_block(act, m, hidden, inter, dtype, dev, replays=20):
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
        for gr in graphs[:2]:
            gr.replay()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(replays):
            graphs[i % len(graphs)].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * per_graph)
    us_fused = timed(fused)
    us_unfused = timed(unfused)
    alg = (width * hidden + hidden * inter) * (0.5 + 4 / 128) + 2 * m * (hidden + width + width + hidden) + 2 * hidden
    del pool, packs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"us_fused": round(us_fused, 3), "us_unfused_torch_activation": round(us_unfused, 3),
            "fused_GBps": round(alg / (us_fused * 1e-6) / 1e9, 1)}


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


# HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
# `bench.py --traffic-probe` (FETCH_SIZE, then WRITE_SIZE), scaled by what the
# same counters read for an elementwise kernel of known size.  The summary
# records a hash of the kernel's sources; a changed kernel reports null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_gate_up_m1_traffic.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "weight_only_int4_rtn_amd", "csrc", f) for f in ("gemv.hip", "common.h")]


def kernel_source_hash() -> str:
    import hashlib
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
    layers, _ = build_pool([c], dev)
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


GEMM_PROBE_CASE = "c4_m1024_k2048_n32768"


def gemm_probe(dev):
    """Launches for the stall-counter runs: the M = 1024 prefill GEMM (K 2048,
    N 32768, fp16 with bias) 8 times over distinct weight copies."""
    import torch

    import synth
    import weight_only_int4_rtn_amd as w4
    c = synth.case_by_name(GEMM_PROBE_CASE)
    layers, _ = build_pool([c], dev)
    x = synth.make_x(c).to(dev)
    bias = synth.make_bias(c).to(dev) if c.bias else None
    y = torch.empty((c.m, c.n), dtype=c.torch_dtype, device=dev)
    ws = torch.zeros(max(w4.workspace_bytes(c.m, c.n, c.k), 16), dtype=torch.uint8, device=dev)
    for i in range(8):
        w4.linear(x, layers[i % len(layers)][0], c.n, bias, out=y, workspace=ws)
    torch.cuda.synchronize()
    log(f"gemm probe: 8 launches of {c.name} on the {w4.choose_path(c.m, c.n, c.k).name} path")


# Stall counters of the GEMM (two rocprofv3 --pmc passes of --gemm-probe):
# SQ_*_CYCLES wave counters count quad-cycles (4 clocks); the MFMA busy
# counter counts clocks summed over the 1024 SIMDs.
SQ_PASSES = (
    ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
     "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"),
    ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
     "SQ_ACTIVE_INST_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM"),
)


def summarize_sq(dbs):
    """Markdown summary of the GEMM's SQ counters from the counter databases
    of --gemm-probe: mean per dispatch (first dispatch dropped), per-wave
    counts, and the shares of a wave's lifetime spent issuing, waiting on
    its counters or a barrier, and waiting to issue."""
    vals = {}
    name = None
    for db in dbs:
        rows = _rocpd_rows(db, "select dispatch_id, kernel_name, counter_name, value from counters_collection")
        per = {}
        for d, kname, cname, v in rows:
            if "gemm" not in kname:
                continue
            name = kname.split("(")[0]
            per.setdefault(cname, {}).setdefault(d, 0.0)
            per[cname][d] += v
        for cname, byd in per.items():
            v = [byd[d] for d in sorted(byd)]
            v = v[1:] if len(v) > 1 else v
            vals[cname] = sum(v) / len(v)
    if not vals:
        raise SystemExit("no GEMM dispatch in the counter databases")
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
    import statistics
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


def cpu_baseline(cases, target_seconds=12.0):
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only the launches the HBM counter runs measure (see TRAFFIC_FILE)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only the launches the GEMM stall-counter runs measure (8 launches of the M = 1024 GEMM)")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DB",
                    help="print the SQ counter summary of --gemm-probe counter databases and exit")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace database and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write TRAFFIC_FILE from the two counter databases of --traffic-probe and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq))
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
        gemm_probe(dev)
        return

    # --- decode step (M = 1) --------------------------------------------------
    cases = decode_cases()
    dominant = 2  # gate_up: the largest stream
    log(f"decode workload: {[c.name for c in cases]}")
    dec = run_workload(cases, dev, args.steps, args.warmup, dominant)
    ms, dom_ms = dec["ms"], dec["dom_ms"]
    step_bytes = sum(c.alg_bytes() for c in cases)
    value = step_bytes / (ms * 1e-3) / 1e9
    dom = cases[dominant]
    dom_gbs = dom.alg_bytes() / (dom_ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.2f} us/step (graph replay), {value:.1f} GB/s; eager {dec['eager_ms'] * 1e3:.1f} us/step; "
        f"gate_up {dom_ms * 1e3:.2f} us/launch, {dom_gbs:.1f} GB/s")

    # --- prefill (M = 1024) ---------------------------------------------------
    pcases = prefill_cases()
    pdom = 1  # N = 32768: the largest GEMM
    log(f"prefill workload: {[c.name for c in pcases]}")
    pre = run_workload(pcases, dev, args.prefill_steps, 5, pdom)
    pms, pdom_ms = pre["ms"], pre["dom_ms"]
    pflops = sum(c.flops() for c in pcases)
    ptf = pflops / (pms * 1e-3) / 1e12
    pd = pcases[pdom]
    pd_tf = pd.flops() / (pdom_ms * 1e-3) / 1e12
    log(f"prefill: {pms * 1e3:.1f} us/step, {ptf:.1f} TFLOP/s; N=32768 {pdom_ms * 1e3:.1f} us, {pd_tf:.1f} TFLOP/s")
    load = dec["load"]

    # --- FFN blocks with the activation fused into the down projection ------
    log("ffn blocks")
    ffn = {
        "swiglu_m1": {"workload": "M=1 bf16: [up | gate] 2048x32768, down 16384x2048 with up*silu(gate) fused",
                      **ffn_block(w4.Act.SWIGLU, 1, 2048, 16384, torch.bfloat16, dev)},
        "gelu_m50": {"workload": "M=50 bf16: up 1024x4096, down 4096x1024 (+bias) with tanh-GELU fused",
                     **ffn_block(w4.Act.GELU_TANH, 50, 1024, 4096, torch.bfloat16, dev)},
    }
    log(f"ffn: {ffn}")

    # --- the same decode step with INT8 weights (W8A16) ----------------------
    log("w8a16 decode workload")
    w8 = run_workload(cases, dev, args.steps, args.warmup, dominant, bits=8, eager=False)
    w8_bytes = sum(alg_bytes(c, 8) for c in cases)
    w8_gbs = w8_bytes / (w8["ms"] * 1e-3) / 1e9
    w8_dom_gbs = alg_bytes(dom, 8) / (w8["dom_ms"] * 1e-3) / 1e9
    w8a16 = {"workload": "decode layer M=1 as above with int8 g128 weights (amax/127)",
             "GBps": round(w8_gbs, 2), "ms_per_step": round(w8["ms"], 5), "bytes_per_step": w8_bytes,
             "pct_hbm_peak": round(100 * w8_gbs / HBM_PEAK_GBS, 2),
             "roofline": {"bound": "hbm", "achieved": round(w8_dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(w8_dom_gbs / HBM_PEAK_GBS, 4),
                          "kernel": f"{w4.choose_path(1, dom.n, dom.k, 8).name} int8 {dom.name}",
                          "avg_launch_us": round(w8["dom_ms"] * 1e3, 3), "bytes_per_launch": alg_bytes(dom, 8)}}
    pre8 = run_workload(pcases, dev, 20, 3, pdom, bits=8, eager=False)
    p8tf = pflops / (pre8["ms"] * 1e-3) / 1e12
    p8d_tf = pd.flops() / (pre8["dom_ms"] * 1e-3) / 1e12
    w8a16["m1024"] = {"workload": "prefill M=1024 fp16 with bias as above, int8 g128 weights",
                      "tflops": round(p8tf, 2), "ms_per_step": round(pre8["ms"], 4),
                      "pct_mfma_peak": round(100 * p8tf / MFMA_PEAK_TFLOPS, 2),
                      "roofline": {"bound": "mfma", "achieved": round(p8d_tf, 2), "peak": MFMA_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(p8d_tf / MFMA_PEAK_TFLOPS, 4),
                                   "kernel": f"{w4.choose_path(pd.m, pd.n, pd.k, 8).name} int8 {pd.name}",
                                   "avg_launch_us": round(pre8["dom_ms"] * 1e3, 3)}}
    log(f"w8a16: {w8a16}")

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
                f"steps replayed as HIP graphs of {dec['steps_per_graph']} consecutive layers)",
        "config": {"workload": "decode layer M=1: qkv 2048x2560, o 2048x2048, gate_up 2048x32768, "
                               "down 16384x2048; bf16 x, int4 g128 weights",
                   "m": 1, "bytes_per_step": step_bytes, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "kernel_path": w4.choose_path(1, 2048, 2048).name,
                   "eager_ms_per_step": round(dec["eager_ms"], 4)},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "kernel": f"{w4.choose_path(1, dom.n, dom.k).name} {dom.name}",
                     "avg_launch_us": round(dom_ms * 1e3, 3), "bytes_per_launch": dom.alg_bytes()},
        "m1024": {"workload": "prefill M=1024 fp16 with bias: K2048xN2560, K2048xN32768, K16384xN2048",
                  "tflops": round(ptf, 2), "ms_per_step": round(pms, 4),
                  "pct_mfma_peak": round(100 * ptf / MFMA_PEAK_TFLOPS, 2),
                  "roofline": {"bound": "mfma", "achieved": round(pd_tf, 2), "peak": MFMA_PEAK_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(pd_tf / MFMA_PEAK_TFLOPS, 4),
                               "kernel": f"{w4.choose_path(pd.m, pd.n, pd.k).name} {pd.name}",
                               "avg_launch_us": round(pdom_ms * 1e3, 3)}},
        "ffn": ffn,
        "w8a16": w8a16,
        "load": {"rows": "quantize + pack, decode layer weights",
                 "GBps": round(load["bytes"] / load["seconds"] / 1e9, 2) if load["seconds"] else None,
                 "shard_GBps": shard_rate(dev),
                 "update": update_rate(dev),
                 "shard": "8 row shards of gate_up 32768x2048 and 8 column shards of down 2048x16384, "
                          "packed to packed, eager launches"},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(cases)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
