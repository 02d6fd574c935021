"""GPU linear layer against the CPU oracle.

  * exact-arithmetic cases: integer codes with scale 2^-3 and small integer
    activations make every partial sum exact in FP32 in any order, so each
    kernel path must return the correctly rounded exact result bit for bit
    (a misplaced nibble, scale, row or split fails exactly);
  * random cases at sizes the oracle finishes quickly, spanning several
    tiles with ragged tails, for every kernel path and both dtypes;
  * the 36 workload cases at full size through the automatic path, compared
    elementwise where the oracle is cheap and on sampled outputs otherwise.
Tolerance (elementwise and mean relative) is defined in tests/gpu_util.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bits, check_close, require_gpu, row_max_dequant, say, tag, to_rne16

pytestmark = pytest.mark.gpu

PATHS = ["GEMV", "MGEMV", "SKINNY", "GEMM", "GEMM_STREAMK"]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def w4():
    import weight_only_int4_rtn_amd as m
    return m


def prepare(w_cpu: torch.Tensor, dev):
    """Quantize on the GPU (checked byte-exact elsewhere) and with the oracle."""
    lib = w4()
    codes, scales = lib.quantize(w_cpu.to(dev))
    packed = lib.pack(codes, scales)
    q, s = oracle.quantize(w_cpu.numpy())
    return packed, q, s


def run(x, packed, n, bias=None, path="AUTO"):
    lib = w4()
    y = lib.linear(x, packed, n, bias, path=lib.Path[path])
    torch.cuda.synchronize()
    return y


def exact_case(m, n, k, seed, dtype, with_bias):
    rng = np.random.default_rng(seed)
    qi = rng.integers(-7, 8, size=(n, k), dtype=np.int8)
    qi[:, ::128] = 7 * np.where(rng.random((n, k // 128)) < 0.5, 1, -1)
    w = torch.from_numpy((qi * 2.0 ** -3).astype(np.float32))
    x = torch.from_numpy(rng.integers(-4, 5, size=(m, k)).astype(np.float32)).to(dtype)
    b = torch.from_numpy(rng.integers(-9, 10, size=n).astype(np.float32)).to(dtype) if with_bias else None
    return w, x, b


# (1, 48, 2176): a 17-group K, the shortest split on 8 waves (3 chunks for
# some waves, 2 for others); (1, 40, 8192): two 8-wave splits; (1, 72,
# 32896): nine splits, the last holding one group; (6, 2056, 16384): two
# 8-wave splits of 64 groups on the MFMA small-M path, and on the v_dot2
# path a 4-row and a 2-row block of 8-wave splits of 32, ragged last tile.
EXACT_SHAPES = [(1, 16, 128), (2, 40, 384), (3, 1000, 2048), (4, 2056, 16384), (5, 72, 256),
                (1, 48, 2176), (1, 40, 8192), (1, 72, 32896), (6, 2056, 16384),
                (17, 130, 640), (33, 64, 1152), (63, 130, 512), (64, 2048, 8192), (65, 40, 256),
                (130, 100, 1152), (255, 72, 384), (257, 136, 256)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", EXACT_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in EXACT_SHAPES])
def test_exact_arithmetic_bit_exact(dev, path, dtype, m, n, k):
    w, x, b = exact_case(m, n, k, seed=m * 7 + n + k, dtype=dtype, with_bias=(m % 2 == 1))
    say(f"exact case path={path} dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare(w, dev)
    assert np.all(s == np.float32(2.0 ** -3))
    y = run(x.to(dev), packed, n, b.to(dev) if b is not None else None, path)
    y_ref = oracle.linear(bits(x), tag(dtype), q, s, bits(b) if b is not None else None)
    want = to_rne16(y_ref, dtype)
    got = y.cpu().to(torch.float64).numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}: got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


# GEMM tilings the planner picks by shape: 256 x 256 tiles with ragged M and
# N, a K split whose parts hold odd and even group counts, a single group
# (LDS-staged epilogue), a row stride that is not a multiple of 8 (direct
# epilogue); and 128 x 256 tiles, one group deep and split; 256 x 256
# tiles over a long K split in six parts of 17 groups and one of 11; 64 x 256
# tiles over a short K, split in two (5 + 4 groups) and unsplit.
# Exact arithmetic, checked bit for bit on whole rows and columns (first,
# last, either side of a tile edge).
GEMM_TILE_SHAPES = [(513, 16424, 1152), (769, 12296, 128), (300, 4104, 640), (1000, 2056, 2176),
                    (512, 32772, 256), (1000, 2056, 14464), (100, 16136, 1152), (1000, 4104, 1024)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", GEMM_TILE_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in GEMM_TILE_SHAPES])
def test_gemm_tilings_bit_exact(dev, dtype, m, n, k):
    w, x, b = exact_case(m, n, k, seed=m + n + k, dtype=dtype, with_bias=True)
    say(f"gemm tiling case dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare(w, dev)
    y = run(x.to(dev), packed, n, b.to(dev), "GEMM").cpu().to(torch.float64).numpy()
    edge_rows = sorted({0, 63, 64, 127, 128, 255, 256, m - 2, m - 1} & set(range(m)))
    edge_cols = sorted({0, 15, 16, 255, 256, n - 17, n - 1} & set(range(n)))
    rows = np.concatenate([np.repeat(edge_rows, n), np.tile(np.arange(m), len(edge_cols))])
    cols = np.concatenate([np.tile(np.arange(n), len(edge_rows)), np.repeat(edge_cols, m)])
    y_ref = oracle.linear_entries(bits(x), tag(dtype), q, s, bits(b), rows, cols)
    want = to_rne16(y_ref, dtype)
    got = y[rows, cols]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} mismatches, first at row {rows[bad[0]]} col {cols[bad[0]]}: "
                           f"got {got[bad[0]]} want {want[bad[0]]}")


# M = 1 plans of the v_dot2 kernel with more than 4 chunks per wave (issued
# 4 ahead of the chunk computed): 16 chunks per wave unsplit (>= 256 row
# tiles), ragged last tile; two splits of 64 + 63 groups (8 chunks per wave,
# the last wave's last chunk past the split); 257 groups in five splits of
# 64 (a tree of three levels, the last split one group).  Exact arithmetic,
# every output bit for bit.
GEMV_SHAPES = [(1, 4104, 16384, 8, 1, 128), (1, 2056, 16256, 8, 2, 64), (1, 1000, 32896, 8, 5, 64)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k,waves,splits,gps", GEMV_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k, *_ in GEMV_SHAPES])
def test_gemv_plans_bit_exact(dev, dtype, m, n, k, waves, splits, gps):
    lib = w4()
    plan = lib.explain(m, n, k, path=lib.Path.GEMV)
    assert (plan["waves"], plan["splits"], plan["groups_per_split"]) == (waves, splits, gps), plan
    w, x, b = exact_case(m, n, k, seed=m + 5 * n + k, dtype=dtype, with_bias=True)
    say(f"gemv plan case dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare(w, dev)
    y = run(x.to(dev), packed, n, b.to(dev), "GEMV")
    want = to_rne16(oracle.linear(bits(x), tag(dtype), q, s, bits(b)), dtype)
    got = y.cpu().to(torch.float64).numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}: got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


# Small-M MFMA plans: x operands loaded with each chunk (M > 4) on 8 waves of
# 8 chunks in two K splits (one exchange level), ragged last row tile; the
# same with a last split one group short and M odd; 4 waves unsplit at M =
# 16; 8 waves of 4 chunk slots over 24 groups (some slots idle); x staged in
# LDS (M = 3) split in four; M = 3 on a small layer (x with the chunks); 63
# row tiles split in four to fill the chip.  Exact arithmetic, every output.
MGEMV_SHAPES = [(8, 2056, 16384, 8, 2, 64), (13, 2056, 16256, 8, 2, 64), (16, 2040, 2048, 4, 1, 16),
                (6, 2056, 3072, 8, 1, 24), (3, 2056, 16384, 8, 4, 32), (3, 2056, 2048, 4, 1, 16),
                (16, 1000, 4096, 4, 4, 8)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k,waves,splits,gps", MGEMV_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k, *_ in MGEMV_SHAPES])
def test_mgemv_plans_bit_exact(dev, dtype, m, n, k, waves, splits, gps):
    lib = w4()
    plan = lib.explain(m, n, k, path=lib.Path.MGEMV)
    assert (plan["waves"], plan["splits"], plan["groups_per_split"]) == (waves, splits, gps), plan
    w, x, b = exact_case(m, n, k, seed=m + 7 * n + k, dtype=dtype, with_bias=True)
    say(f"mgemv plan case dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare(w, dev)
    y = run(x.to(dev), packed, n, b.to(dev), "MGEMV")
    want = to_rne16(oracle.linear(bits(x), tag(dtype), q, s, bits(b)), dtype)
    got = y.cpu().to(torch.float64).numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}: got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


# Mid-M plans without a fused activation (x slice whole in LDS): 32-row
# blocks on 8 waves (128 columns per workgroup), unsplit, ragged last tile and
# rows past M, and split in eight (finished in the launch through 128-column
# slots); 16-row blocks with a K split finished in the launch whose last part
# is one group short; a small layer in 16-row blocks, M not a multiple of 16,
# split in four; a small layer split in eight parts of 8 groups (512
# workgroups).  Exact arithmetic, whole rows and columns at the edges.
SKINNY_SHAPES = [(37, 16376, 2048, 8, 1), (61, 2040, 16384, 8, 8), (13, 2056, 16256, 4, 8),
                 (61, 1000, 4096, 4, 4), (64, 1040, 8192, 4, 8)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k,waves,splits", SKINNY_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k, _, _ in SKINNY_SHAPES])
def test_skinny_plans_bit_exact(dev, dtype, m, n, k, waves, splits):
    lib = w4()
    plan = lib.explain(m, n, k, path=lib.Path.SKINNY)
    assert (plan["waves"], plan["splits"]) == (waves, splits), plan
    w, x, b = exact_case(m, n, k, seed=m + 3 * n + k, dtype=dtype, with_bias=True)
    say(f"skinny plan case dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare(w, dev)
    y = run(x.to(dev), packed, n, b.to(dev), "SKINNY").cpu().to(torch.float64).numpy()
    edge_rows = sorted({0, 15, 16, 31, 32, m - 2, m - 1} & set(range(m)))
    edge_cols = sorted({0, 15, 16, 63, 64, 127, 128, n - 17, n - 9, n - 1} & set(range(n)))
    rows = np.concatenate([np.repeat(edge_rows, n), np.tile(np.arange(m), len(edge_cols))])
    cols = np.concatenate([np.tile(np.arange(n), len(edge_rows)), np.repeat(edge_cols, m)])
    y_ref = oracle.linear_entries(bits(x), tag(dtype), q, s, bits(b), rows, cols)
    want = to_rne16(y_ref, dtype)
    got = y[rows, cols]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} mismatches, first at row {rows[bad[0]]} col {cols[bad[0]]}: "
                           f"got {got[bad[0]]} want {want[bad[0]]}")


def test_strided_output_bit_exact(dev):
    """Row stride ldy > n through the C-ABI: every path writes exactly the
    n outputs of each row (the padding keeps its sentinel), bit-exact.
    1024 x 16388 takes the 256 x 256 GEMM tiles with one K split, the
    LDS-staged epilogue and a ragged last 8-column unit."""
    from weight_only_int4_rtn_amd import _binding as B
    m, n, k = 1024, 16388, 256
    ldy = n + 4
    w, x, b = exact_case(m, n, k, seed=5, dtype=torch.bfloat16, with_bias=True)
    packed, q, s = prepare(w, dev)
    xd, bd = x.to(dev), b.to(dev)
    need = max(B.workspace_bytes(m, n, k), B.explain(m, n, k, path=B.Path.GEMM_STREAMK)["workspace_bytes"])
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    rows = np.array(sorted({0, 1, 255, 256, 511, 1022, 1023}))
    cols = np.array(sorted({0, 7, 8, 255, 256, 16383, 16384, 16385, 16386, 16387}))
    rr, cc = np.meshgrid(rows, cols, indexing="ij")
    want = to_rne16(oracle.linear_entries(bits(x), tag(torch.bfloat16), q, s, bits(b), rr.ravel(), cc.ravel()),
                    torch.bfloat16)
    sentinel = -12352.0  # exact in bf16
    for path in PATHS:
        say(f"strided output path={path} m={m} n={n} k={k} ldy={ldy}")
        ybuf = torch.full((m, ldy), sentinel, dtype=torch.bfloat16, device=dev)
        st = B.lib().w4a16_linear_with_path(int(B.Path[path]), B._ptr(xd), B._act_tag(xd.dtype), m, k, k,
                                            B._ptr(packed), n, B._ptr(bd), B._ptr(ybuf), ldy, B._ptr(ws),
                                            ws.numel(), B._stream(dev))
        torch.cuda.synchronize()
        assert st == 0, (path, B.status_string(st))
        yc = ybuf.cpu().to(torch.float64).numpy()
        assert np.all(yc[:, n:] == sentinel), path
        got = yc[rr.ravel(), cc.ravel()]
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, f"{path}: {bad.size} mismatches, first at {rr.ravel()[bad[0]]},{cc.ravel()[bad[0]]}"


# Calls of different shapes and paths sharing one zero-filled workspace, in an
# order where a later call's partial sums land where an earlier call's could
# have been: every result bit-exact, and the 1 MiB exchange-slot header zero
# again after every call.  Small-M splits: GEMV into 4, 3 (a tree with an odd
# child), 8 (too many slots: partial sums and the reduce kernel) and 5 parts;
# MGEMV into 2 (x operands with the chunks), 8 (the same, too many slots:
# partial sums) and 8 parts (x staged in LDS, three tree levels); stream-K
# GEMMs whose runs share tiles (their tile counters sit in the same header).
SYNC_HEADER = 1 << 20
SHARED_WS_CALLS = [("GEMV", 1, 2048, 16384), ("SKINNY", 50, 1000, 4096), ("GEMV", 3, 40, 12288),
                   ("MGEMV", 8, 2048, 16384), ("GEMM", 300, 4104, 640), ("GEMV", 4, 4688, 32768),
                   ("MGEMV", 16, 1200, 65536), ("GEMM_STREAMK", 130, 2056, 2176), ("GEMV", 2, 100, 20480),
                   ("MGEMV", 4, 1024, 16384), ("GEMM_STREAMK", 97, 4104, 4096), ("GEMV", 1, 2048, 16384)]


def test_shared_workspace_header_stays_clear(dev):
    from weight_only_int4_rtn_amd import _binding as B
    lib = w4()
    need = max(max(B.workspace_bytes(m, n, k), B.explain(m, n, k, path=B.Path[p])["workspace_bytes"])
               for p, m, n, k in SHARED_WS_CALLS)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    splits_seen = 0
    for i, (path, m, n, k) in enumerate(SHARED_WS_CALLS):
        say(f"shared workspace call {i}: path={path} m={m} n={n} k={k}")
        w, x, b = exact_case(m, n, k, seed=40 + i, dtype=torch.bfloat16, with_bias=(i % 2 == 0))
        packed, q, s = prepare(w, dev)
        plan = B.explain(m, n, k, path=B.Path[path])
        splits_seen += plan["splits"] > 1
        if path == "GEMM_STREAMK":
            assert plan["stream_k"] == 1 and plan["splits"] > 1, plan
        y = lib.linear(x.to(dev), packed, n, b.to(dev) if b is not None else None, path=lib.Path[path],
                       workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:SYNC_HEADER].count_nonzero()) == 0, f"call {i}: exchange-slot header not left zero"
        want = to_rne16(oracle.linear(bits(x), tag(torch.bfloat16), q, s, bits(b) if b is not None else None),
                        torch.bfloat16)
        got = y.cpu().to(torch.float64).numpy()
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"call {i} ({path} {m}x{n}x{k}): {len(bad)} mismatches, first {bad[:3].tolist()}"
    assert splits_seen >= 10


def random_case(m, n, k, seed, dtype, with_bias):
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(n, k, generator=g) * 0.02
    mask = torch.rand(n, k, generator=g) < 0.01
    w = torch.where(mask, torch.randn(n, k, generator=g) * 0.2, w)
    w[:, :128][::7] = 0.0  # some all-zero groups
    x = torch.randn(m, k, generator=g)
    x[:, ::64] *= 10.0
    x = x.to(dtype)
    b = (torch.randn(n, generator=g) * 0.01).to(dtype) if with_bias else None
    return w, x, b


RANDOM_SHAPES = [(1, 24, 256), (2, 1000, 1024), (3, 100, 4096), (4, 520, 2048), (1, 2048, 16384),
                 (6, 200, 640), (16, 1000, 2048), (31, 77, 1280), (50, 1024, 4096), (64, 264, 3072),
                 (100, 520, 1024), (257, 130, 512)]


@pytest.mark.parametrize("path", PATHS + ["AUTO"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", RANDOM_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in RANDOM_SHAPES])
def test_random_within_tolerance(dev, path, dtype, m, n, k):
    w, x, b = random_case(m, n, k, seed=1000 + m + n + k, dtype=dtype, with_bias=(n % 2 == 0))
    say(f"random case path={path} dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare(w, dev)
    y = run(x.to(dev), packed, n, b.to(dev) if b is not None else None, path)
    y_ref = oracle.linear(bits(x), tag(dtype), q, s, bits(b) if b is not None else None)
    xnorm = np.linalg.norm(x.to(torch.float64).numpy(), axis=1)[:, None]
    wmax = row_max_dequant(q, s)[None, :]
    check_close(y.cpu().numpy() if y.dtype == torch.float32 else y.cpu().to(torch.float64).numpy(),
                y_ref, xnorm, wmax, f"{path} m={m} n={n} k={k}")


def test_leading_dims_and_strided_out(dev):
    lib = w4()
    w, x, b = random_case(6, 48, 256, seed=3, dtype=torch.bfloat16, with_bias=True)
    packed, q, s = prepare(w, dev)
    x3 = x.reshape(2, 3, 256).to(dev)
    y = lib.linear(x3, packed, 48, b.to(dev))
    torch.cuda.synchronize()
    assert y.shape == (2, 3, 48)
    y2 = run(x.to(dev), packed, 48, b.to(dev))
    assert torch.equal(y.reshape(6, 48), y2)


def test_results_are_deterministic(dev):
    c = synth.case_by_name("c3_down_m4_k16384_n2048")
    packed, q, s = prepare(synth.make_weight(c), dev)
    x = synth.make_x(c).to(dev)
    say("determinism: c3 down m4")
    for path in PATHS:
        a = run(x, packed, c.n, path=path)
        b = run(x, packed, c.n, path=path)
        assert torch.equal(a, b), path


# --- the 36 workload cases at full size --------------------------------------

_weights = {}


def workload_weight(c, dev):
    key = (c.config, c.shape_index)
    if key not in _weights:
        _weights.clear()  # keep at most one layer's weights resident
        w = synth.make_weight(c)
        packed, q, s = prepare(w, dev)
        _weights[key] = (packed, q, s, row_max_dequant(q, s))
    return _weights[key]


FULL_LIMIT = 1 << 31  # m*n*k above which outputs are sampled


@pytest.mark.parametrize("name", [c.name for c in synth.all_cases()])
def test_workload_case(dev, name):
    c = synth.case_by_name(name)
    say(f"workload case {name}: m={c.m} k={c.k} n={c.n} {c.dtype} bias={c.bias}")
    packed, q, s, wmax = workload_weight(c, dev)
    x = synth.make_x(c)
    b = synth.make_bias(c)
    y = run(x.to(dev), packed, c.n, b.to(dev) if b is not None else None).cpu().to(torch.float64).numpy()
    xb = bits(x)
    bb = bits(b) if b is not None else None
    xnorm = np.linalg.norm(x.to(torch.float64).numpy(), axis=1)
    if c.m * c.n * c.k <= FULL_LIMIT:
        y_ref = oracle.linear(xb, tag(c.torch_dtype), q, s, bb)
        check_close(y, y_ref, xnorm[:, None], wmax[None, :], name)
    else:
        rng = np.random.default_rng(7)
        rows = np.concatenate([rng.integers(0, c.m, 4096), [0, c.m - 1, c.m - 1, 0]])
        cols = np.concatenate([rng.integers(0, c.n, 4096), [0, c.n - 1, 0, c.n - 1]])
        y_ref = oracle.linear_entries(xb, tag(c.torch_dtype), q, s, bb, rows, cols)
        check_close(y[rows, cols], y_ref, xnorm[rows], wmax[cols], name)


def test_concurrent_streams_separate_workspaces(dev):
    """Calls with K splits finished through the exchange slots, issued on two
    streams at once, each with the binding's own workspace for its stream,
    equal the same calls made one after the other, bit for bit."""
    lib = w4()
    g = torch.Generator().manual_seed(77)
    layers = []
    for n, k in ((2048, 16384), (1040, 16384)):
        w = torch.randn(n, k, generator=g) * 0.02
        c, s = lib.quantize(w.to(dev))
        layers.append((lib.pack(c, s), n, k))
    xs = [torch.randn(m, k, generator=g).to(torch.bfloat16).to(dev) for m, (_, _, k) in zip((1, 6), layers)]
    want = [lib.linear(x, p, n) for x, (p, n, _) in zip(xs, layers)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    say("two streams, 8 rounds of split-K calls each")
    outs = [[], []]
    for _ in range(8):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                p, n, _ = layers[i]
                outs[i].append(lib.linear(xs[i], p, n))
    torch.cuda.synchronize()
    for i in range(2):
        for y in outs[i]:
            assert torch.equal(y, want[i]), f"stream {i}"
