"""The linear layer's calls captured in a HIP graph (torch.cuda.graph) and
replayed equal the eager calls bit for bit: the calls allocate nothing,
synchronise nothing and record no memset, and the K-split exchange slots are
left zero by every replay.  Replays are interleaved with eager work and
synchronisations, and every replay is checked."""
import numpy as np
import pytest
import torch

from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

# (m, n, k, act, bits, path): GEMV with a K split finished through the
# exchange slots, MGEMV split, SKINNY split + reduce kernel, GEMM, a fused
# SwiGLU input, the GEMM path with a materialised GELU input; INT8 weights on
# the GEMV (eight-part split), MGEMV (split through the exchange slots),
# SKINNY and 256 x 256 GEMM paths; stream-K GEMMs whose runs share tiles
# (tile counters in the header, INT4 and INT8, one with a GELU input)
CALLS = [(1, 2048, 16384, "NONE", 4, "AUTO"), (6, 520, 8192, "NONE", 4, "AUTO"),
         (50, 1000, 4096, "NONE", 4, "AUTO"), (300, 2056, 1152, "NONE", 4, "GEMM"),
         (1, 1024, 4096, "SWIGLU", 4, "AUTO"), (256, 512, 1024, "GELU_TANH", 4, "GEMM"),
         (1, 2048, 16384, "NONE", 8, "AUTO"), (4, 2048, 16384, "NONE", 8, "MGEMV"),
         (50, 1000, 4096, "SWIGLU", 8, "AUTO"), (300, 2056, 1152, "GELU_TANH", 8, "GEMM"),
         (130, 2056, 2176, "NONE", 4, "GEMM_STREAMK"), (97, 4104, 4096, "GELU_TANH", 4, "GEMM_STREAMK"),
         (130, 2056, 2176, "NONE", 8, "GEMM_STREAMK")]


def test_graph_replays_equal_eager(dev=None):
    dev = require_gpu()
    import weight_only_int4_rtn_amd as w4
    g = torch.Generator().manual_seed(11)
    setups = []
    ws_bytes = 16
    for m, n, k, act, nbits, path in CALLS:
        w = torch.randn(n, k, generator=g) * 0.02
        width = 2 * k if act == "SWIGLU" else k
        x = torch.randn(m, width, generator=g).to(torch.bfloat16).to(dev)
        b = (torch.randn(n, generator=g) * 0.01).to(torch.bfloat16).to(dev)
        if nbits == 8:
            c, s = w4.quantize_int8(w.to(dev))
            p = w4.pack_int8(c, s)
        else:
            c, s = w4.quantize(w.to(dev))
            p = w4.pack(c, s)
        y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        setups.append((m, n, k, w4.Act[act], nbits, w4.Path[path], x, p, b, y))
        ws_bytes = max(ws_bytes, w4.workspace_bytes(m, n, k, w4.Act[act], nbits),
                       w4.explain(m, n, k, w4.Act[act], w4.Path[path], nbits)["workspace_bytes"])
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)

    def run():
        for m, n, k, act, nbits, path, x, p, b, y in setups:
            w4.linear(x, p, n, b, out=y, workspace=ws, act=act, bits=nbits, path=path)

    run()
    torch.cuda.synchronize()
    eager = [s[-1].clone() for s in setups]
    for s in setups:
        s[-1].fill_(0.0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"graph replay {rep}")
        for s in setups:
            s[-1].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, s in enumerate(setups):
            assert torch.equal(s[-1], eager[i]), f"replay {rep}, call {i} {CALLS[i]}"
        assert int(ws[:1 << 20].count_nonzero()) == 0, f"replay {rep}: exchange slots not left zero"
        # eager work between replays (same workspace, other shapes)
        w4.linear(setups[2][6], setups[2][7], setups[2][1], workspace=ws)
        torch.cuda.synchronize()


def test_two_graphs_without_workspace():
    """Calls that need no workspace capture with workspace=None: two graphs
    captured one after the other, each replayed several times between eager
    work, equal the eager results bit for bit.  (A call that needs a
    workspace is refused under capture without one: a host check, tested in
    test_boundary.py.)"""
    dev = require_gpu()
    import weight_only_int4_rtn_amd as w4
    g = torch.Generator().manual_seed(12)
    # (m, n, k): GEMV and MGEMV at two groups, SKINNY, GEMM - no K split anywhere
    shapes = [[(1, 4096, 256), (3, 1040, 128)], [(40, 2056, 256), (300, 512, 128)]]
    setups = []
    for group in shapes:
        calls = []
        for m, n, k in group:
            assert w4.workspace_bytes(m, n, k) == 0
            c, s = w4.quantize((torch.randn(n, k, generator=g) * 0.02).to(dev))
            x = torch.randn(m, k, generator=g).to(torch.bfloat16).to(dev)
            calls.append((x, w4.pack(c, s), n, torch.empty(m, n, dtype=torch.bfloat16, device=dev)))
        setups.append(calls)
    eager = []
    for calls in setups:
        eager.append([w4.linear(x, p, n).clone() for x, p, n, _ in calls])
    torch.cuda.synchronize()
    graphs = []
    for calls in setups:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for x, p, n, y in calls:
                w4.linear(x, p, n, out=y)
        graphs.append(gr)
    torch.cuda.synchronize()
    for rep in range(3):
        for gi, (gr, calls) in enumerate(zip(graphs, setups)):
            say(f"graph {gi} replay {rep}")
            for *_, y in calls:
                y.fill_(float("nan"))
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            for ci, (*_, y) in enumerate(calls):
                assert torch.equal(y, eager[gi][ci]), f"graph {gi} replay {rep} call {ci}"
            w4.linear(setups[0][0][0], setups[0][0][1], setups[0][0][2])  # eager work between replays
