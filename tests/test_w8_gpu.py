"""W8A16 (INT8 weights) on the GPU against the CPU oracle.

  * quantization: codes and scales byte-equal to ``oracle.quantize_int8`` on
    workload weights and edge cases (ties, zero and -0 groups, subnormal and
    underflowing scales, huge magnitudes, 16-bit and strided weights);
  * packing: round trip on arbitrary bytes (code -128 included), and the
    packed bytes equal the layout documented in the library's headers,
    built here from that description;
  * the linear layer on the four INT8 kernel paths (GEMV, the MFMA small-M
    kernel, SKINNY, and the 256 x 256 GEMM) and the automatic choice: exact-arithmetic cases bit for bit (integer codes with
    scale 2^-3 and small integer activations make every partial sum exact),
    random ragged cases within the tolerance of tests/gpu_util.py, fused
    activations, K splits through the exchange slots and through partial
    sums, and the workload shapes at full size on sampled outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bits, check_close, require_gpu, row_max_dequant, say, tag, to_rne16

pytestmark = pytest.mark.gpu

PATHS8 = ["GEMV", "MGEMV", "SKINNY", "GEMM", "GEMM_STREAMK", "AUTO"]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def w4():
    import weight_only_int4_rtn_amd as m
    return m


def oracle_q8(w_cpu: torch.Tensor):
    if w_cpu.dtype == torch.float32:
        return oracle.quantize_int8(w_cpu.numpy())
    return oracle.quantize_int8(bits(w_cpu), tag(w_cpu.dtype))


def gpu_q8(w_dev: torch.Tensor):
    codes, scales = w4().quantize_int8(w_dev)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


# --- quantization --------------------------------------------------------------

Q8_CASES = ["c1_m1_k1024_n1024", "c2_down_m50_k4096_n1024", "c3_down_m1_k16384_n2048",
            "c3_qkv_m1_k2048_n2560", "c5_m1_k2048_n16384"]


@pytest.mark.parametrize("name", Q8_CASES)
def test_quantize_int8_matches_oracle(dev, name):
    c = synth.case_by_name(name)
    say(f"int8 quantize parity: {name} n={c.n} k={c.k}")
    w = synth.make_weight(c)
    codes, scales = gpu_q8(w.to(dev))
    q, s = oracle_q8(w)
    assert np.array_equal(scales.view(np.uint32), s.view(np.uint32)), "scales differ"
    diff = np.flatnonzero(codes != q)
    assert diff.size == 0, f"{diff.size} codes differ, first at {diff[:5]}"


def edge_weights8():
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((40, 1024)) * 0.02).astype(np.float32)
    w[0, :128] = 0.0
    w[0, 0] = 127.0                               # scale 1: exact ties below
    w[0, 1:10] = [0.5, 1.5, 2.5, -2.5, -126.5, 126.5, 63.5, -0.5, 100.5]
    w[1, 128:256] = 0.0                           # all-zero group
    w[2, 256:384] = -0.0                          # negative zeros
    w[3, :128] *= np.float32(1e-39)               # subnormal group
    w[4, 128:256] = 0.0
    w[4, 128] = np.float32(2.0 ** -149) * 2       # amax / 127 underflows to 0
    w[5, 256:384] = 0.0
    w[5, 256] = np.float32(2.0 ** -149) * 127     # scale = smallest subnormal
    w[5, 257] = -np.float32(2.0 ** -149) * 64
    w[6, :] *= np.float32(1e30)                   # huge magnitudes
    w[7, 384:512] = np.float32(0.7) * np.arange(128, dtype=np.float32) / np.float32(254.0)  # half-code steps
    w[8, :] = np.float32(-1.0)                    # constant rows
    w[9, ::2] = -w[9, 1::2]
    return w


def test_quantize_int8_edge_cases(dev):
    w = torch.from_numpy(edge_weights8())
    say("int8 quantize parity: edge cases")
    codes, scales = gpu_q8(w.to(dev))
    q, s = oracle_q8(w)
    assert np.array_equal(scales.view(np.uint32), s.view(np.uint32))
    assert np.array_equal(codes, q)
    assert codes.min() >= -127


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_quantize_int8_16bit_and_strided(dev, dtype):
    rng = np.random.default_rng(6)
    full = torch.from_numpy((rng.standard_normal((24, 640)) * 0.02).astype(np.float32)).to(dtype)
    say(f"int8 quantize parity: {dtype} weights, strided rows")
    codes, scales = gpu_q8(full.to(dev)[:, :512])
    q, s = oracle_q8(full[:, :512].contiguous())
    assert np.array_equal(scales.view(np.uint32), s.view(np.uint32))
    assert np.array_equal(codes, q)


# --- packing -------------------------------------------------------------------


def documented_layout(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The packed INT8 bytes as the layout description states them: chunk
    (t, g) of 2048 code bytes at (t*G + g)*2048; half h, lane L = r + 16 kq,
    word j holds columns 128g + 32(2h + j/2) + 8kq + 4(j%2) + b (byte b) of
    row 16t + r as q + 128; padding rows code 0; scales after the codes, 16
    per chunk."""
    n, k = codes.shape
    T, G = -(-n // 16), k // 128
    u = np.full((T * 16, k), 128, dtype=np.uint8)
    u[:n] = (codes.astype(np.int16) + 128).astype(np.uint8)
    out = np.zeros(T * G * (2048 + 64), dtype=np.uint8)
    for t in range(T):
        for g in range(G):
            base = (t * G + g) * 2048
            for h in range(2):
                for lane in range(64):
                    r, kq = lane % 16, lane // 16
                    for j in range(4):
                        c0 = 128 * g + 32 * (2 * h + j // 2) + 8 * kq + 4 * (j % 2)
                        off = base + 1024 * h + 16 * lane + 4 * j
                        out[off:off + 4] = u[16 * t + r, c0:c0 + 4]
    sc = np.zeros((T * 16, G), dtype=np.float32)
    sc[:n] = scales
    sv = out[T * G * 2048:].view(np.float32)
    for t in range(T):
        for g in range(G):
            sv[(t * G + g) * 16:(t * G + g + 1) * 16] = sc[16 * t:16 * t + 16, g]
    return out


@pytest.mark.parametrize("n,k", [(16, 128), (17, 256), (40, 384)])
def test_pack_int8_matches_documented_layout(dev, n, k):
    rng = np.random.default_rng(n * k)
    codes = rng.integers(-128, 128, size=(n, k), dtype=np.int8)
    scales = rng.standard_normal((n, k // 128)).astype(np.float32)
    say(f"int8 pack layout n={n} k={k}")
    packed = w4().pack_int8(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    torch.cuda.synchronize()
    want = documented_layout(codes, scales)
    got = packed.cpu().numpy()
    assert got.size == want.size == w4().packed_bytes(n, k, bits=8)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:5]}"


@pytest.mark.parametrize("n,k", [(16, 128), (1000, 384), (2056, 1152)])
def test_pack_int8_roundtrip_any_bytes(dev, n, k):
    rng = np.random.default_rng(n + k)
    codes = torch.from_numpy(rng.integers(-128, 128, size=(n, k), dtype=np.int8)).to(dev)
    scales = torch.from_numpy(rng.standard_normal((n, k // 128)).astype(np.float32)).to(dev)
    say(f"int8 pack round trip n={n} k={k}")
    lib = w4()
    packed = lib.pack_int8(codes, scales)
    c2, s2 = lib.unpack_int8(packed, n, k)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes)
    assert torch.equal(s2.view(torch.int32), scales.view(torch.int32))


# --- linear --------------------------------------------------------------------


def prepare8(w_cpu: torch.Tensor, dev):
    lib = w4()
    codes, scales = lib.quantize_int8(w_cpu.to(dev))
    packed = lib.pack_int8(codes, scales)
    q, s = oracle.quantize_int8(w_cpu.numpy())
    return packed, q, s


def run8(x, packed, n, bias=None, path="AUTO", act=None, workspace=None):
    lib = w4()
    y = lib.linear(x, packed, n, bias, path=lib.Path[path], act=act if act is not None else lib.Act.NONE,
                   bits=8, workspace=workspace)
    torch.cuda.synchronize()
    return y


def exact_case8(m, n, k, seed, dtype, with_bias):
    rng = np.random.default_rng(seed)
    qi = rng.integers(-127, 128, size=(n, k)).astype(np.int16)
    qi[:, ::128] = 127 * np.where(rng.random((n, k // 128)) < 0.5, 1, -1)
    w = torch.from_numpy((qi * 2.0 ** -3).astype(np.float32))
    x = torch.from_numpy(rng.integers(-4, 5, size=(m, k)).astype(np.float32)).to(dtype)
    b = torch.from_numpy(rng.integers(-9, 10, size=n).astype(np.float32)).to(dtype) if with_bias else None
    return w, x, b


# GEMV row blocks (m 1..4, 6), K splits of the GEMV (16 groups per
# workgroup: k 2048 one part, 16384 eight parts, 20480 ten) and of SKINNY,
# ragged n and m tails, several m-blocks.
EXACT8_SHAPES = [(1, 16, 128), (2, 40, 384), (3, 1000, 2048), (4, 2056, 16384), (6, 72, 256),
                 (1, 100, 20480), (17, 130, 640), (33, 64, 1152), (63, 130, 512), (64, 2048, 8192),
                 (65, 40, 256), (130, 100, 1152), (257, 136, 256)]


@pytest.mark.parametrize("path", PATHS8)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", EXACT8_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in EXACT8_SHAPES])
def test_int8_exact_arithmetic_bit_exact(dev, path, dtype, m, n, k):
    w, x, b = exact_case8(m, n, k, seed=m * 5 + n + k, dtype=dtype, with_bias=(m % 2 == 1))
    say(f"int8 exact case path={path} dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare8(w, dev)
    assert np.all(s == np.float32(2.0 ** -3))
    y = run8(x.to(dev), packed, n, b.to(dev) if b is not None else None, path)
    want = to_rne16(oracle.linear(bits(x), tag(dtype), q, s, bits(b) if b is not None else None), dtype)
    got = y.cpu().to(torch.float64).numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}: got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}"


# The mid-M direct kernel's 32-row schedule on INT8 weights (8 waves, 128
# columns; each pair's two-half chunks loaded with its x blocks): unsplit,
# ragged last tile, rows past M.  Exact arithmetic, whole rows and columns at
# the edges.
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_int8_skinny_paired_plan_bit_exact(dev, dtype):
    import weight_only_int4_rtn_amd as w4
    m, n, k = 40, 16376, 1024
    plan = w4.explain(m, n, k, path=w4.Path.SKINNY, bits=8)
    assert (plan["waves"], plan["splits"]) == (8, 1), plan
    w, x, b = exact_case8(m, n, k, seed=m + 7 * n + k, dtype=dtype, with_bias=True)
    say(f"int8 skinny paired plan dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare8(w, dev)
    y = run8(x.to(dev), packed, n, b.to(dev), "SKINNY").cpu().to(torch.float64).numpy()
    edge_rows = sorted({0, 15, 16, 31, 32, m - 2, m - 1})
    edge_cols = sorted({0, 15, 16, 127, 128, n - 17, n - 9, n - 1})
    rows = np.concatenate([np.repeat(edge_rows, n), np.tile(np.arange(m), len(edge_cols))])
    cols = np.concatenate([np.tile(np.arange(n), len(edge_rows)), np.repeat(edge_cols, m)])
    want = to_rne16(oracle.linear_entries(bits(x), tag(dtype), q, s, bits(b), rows, cols), dtype)
    got = y[rows, cols]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} mismatches, first at row {rows[bad[0]]} col {cols[bad[0]]}: "
                           f"got {got[bad[0]]} want {want[bad[0]]}")


# The v_dot2 GEMV at M = 1 on INT8 weights: splits of 64 groups on 8 waves
# of 8 two-half chunks (a window of 2 ahead), the last split one group
# short, ragged last tile; 20 groups on 8 waves of 4 chunk slots (some
# idle).  Exact arithmetic, every output.
GEMV8_SHAPES = [(1, 2056, 16256, 8, 2, 64), (1, 1000, 2560, 8, 1, 20)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k,waves,splits,gps", GEMV8_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k, *_ in GEMV8_SHAPES])
def test_int8_gemv_plans_bit_exact(dev, dtype, m, n, k, waves, splits, gps):
    import weight_only_int4_rtn_amd as w4
    plan = w4.explain(m, n, k, path=w4.Path.GEMV, bits=8)
    assert (plan["waves"], plan["splits"], plan["groups_per_split"]) == (waves, splits, gps), plan
    w, x, b = exact_case8(m, n, k, seed=m + 11 * n + k, dtype=dtype, with_bias=True)
    say(f"int8 gemv plan dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare8(w, dev)
    y = run8(x.to(dev), packed, n, b.to(dev), "GEMV").cpu().to(torch.float64).numpy()
    want = to_rne16(oracle.linear(bits(x), tag(dtype), q, s, bits(b)), dtype)
    bad = np.argwhere(y != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


# The eight-wave GEMM on INT8 weights: ragged M and N over 256 x 256 tiles,
# no split (one LDS-staged epilogue), an uneven long-K split (six parts of
# 17 groups and one of 11), a single group, and a K split with odd group
# counts.  Exact arithmetic, bit for bit on whole rows and columns at tile
# edges.
GEMM8_TILE_SHAPES = [(513, 16424, 1152), (1000, 2056, 14464), (769, 12296, 128), (300, 4104, 640)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", GEMM8_TILE_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in GEMM8_TILE_SHAPES])
def test_int8_gemm_tilings_bit_exact(dev, dtype, m, n, k):
    w, x, b = exact_case8(m, n, k, seed=m + n + k + 1, dtype=dtype, with_bias=True)
    say(f"int8 gemm tiling case dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare8(w, dev)
    y = run8(x.to(dev), packed, n, b.to(dev), "GEMM").cpu().to(torch.float64).numpy()
    edge_rows = sorted({0, 127, 128, 255, 256, m - 2, m - 1} & set(range(m)))
    edge_cols = sorted({0, 15, 16, 255, 256, n - 17, n - 1} & set(range(n)))
    rows = np.concatenate([np.repeat(edge_rows, n), np.tile(np.arange(m), len(edge_cols))])
    cols = np.concatenate([np.tile(np.arange(n), len(edge_rows)), np.repeat(edge_cols, m)])
    want = to_rne16(oracle.linear_entries(bits(x), tag(dtype), q, s, bits(b), rows, cols), dtype)
    got = y[rows, cols]
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{bad.size} mismatches, first at row {rows[bad[0]]} col {cols[bad[0]]}: "
                           f"got {got[bad[0]]} want {want[bad[0]]}")


def random_case8(m, n, k, seed, dtype, with_bias, xcols=None):
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(n, k, generator=g) * 0.02
    mask = torch.rand(n, k, generator=g) < 0.01
    w = torch.where(mask, torch.randn(n, k, generator=g) * 0.2, w)
    w[:, :128][::7] = 0.0
    x = torch.randn(m, xcols or k, generator=g)
    x[:, ::64] *= 10.0
    b = (torch.randn(n, generator=g) * 0.01).to(dtype) if with_bias else None
    return w, x.to(dtype), b


RANDOM8_SHAPES = [(1, 24, 256), (2, 1000, 1024), (3, 100, 4096), (4, 520, 2048), (1, 2048, 16384),
                  (5, 200, 640), (16, 1000, 2048), (31, 77, 1280), (50, 1024, 4096), (100, 520, 1024),
                  (257, 130, 512)]


@pytest.mark.parametrize("path", PATHS8)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", RANDOM8_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in RANDOM8_SHAPES])
def test_int8_random_within_tolerance(dev, path, dtype, m, n, k):
    w, x, b = random_case8(m, n, k, seed=2000 + m + n + k, dtype=dtype, with_bias=(n % 2 == 0))
    say(f"int8 random case path={path} dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare8(w, dev)
    y = run8(x.to(dev), packed, n, b.to(dev) if b is not None else None, path)
    y_ref = oracle.linear(bits(x), tag(dtype), q, s, bits(b) if b is not None else None)
    xnorm = np.linalg.norm(x.to(torch.float64).numpy(), axis=1)[:, None]
    check_close(y.cpu().to(torch.float64).numpy(), y_ref, xnorm, row_max_dequant(q, s)[None, :],
                f"int8 {path} m={m} n={n} k={k}")


ACT8_SHAPES = [(1, 520, 2048), (3, 100, 16384), (16, 200, 1024), (50, 1024, 4096)]


@pytest.mark.parametrize("act", ["SWIGLU", "GELU_TANH"])
@pytest.mark.parametrize("path", PATHS8)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", ACT8_SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in ACT8_SHAPES])
def test_int8_fused_activation(dev, act, path, dtype, m, n, k):
    lib = w4()
    a = lib.Act[act]
    xcols = 2 * k if a == lib.Act.SWIGLU else k
    w, x, b = random_case8(m, n, k, seed=3000 + m + n + k, dtype=dtype, with_bias=True, xcols=xcols)
    x = (x.to(torch.float32) * 0.25).to(dtype)
    say(f"int8 fused {act} path={path} dtype={dtype} m={m} n={n} k={k}")
    packed, q, s = prepare8(w, dev)
    y = run8(x.to(dev), packed, n, b.to(dev), path, act=a)
    fn = oracle.ACT_SWIGLU if a == lib.Act.SWIGLU else oracle.ACT_GELU_TANH
    xa = oracle.activate(bits(x), tag(dtype), fn)
    y_ref = oracle.linear(xa, tag(dtype), q, s, bits(b))
    at = torch.from_numpy(xa.view(np.int16)).view(dtype).to(torch.float64).numpy()
    xnorm = np.linalg.norm(at, axis=1)[:, None]
    check_close(y.cpu().to(torch.float64).numpy(), y_ref, xnorm, row_max_dequant(q, s)[None, :],
                f"int8 {act} {path} m={m} n={n} k={k}")


def test_int8_shared_workspace_and_determinism(dev):
    """INT8 K splits (GEMV through the exchange slots and through partial
    sums, SKINNY through partial sums) sharing one workspace with INT4 calls:
    bit-exact, header left zero, repeat calls identical."""
    from weight_only_int4_rtn_amd import _binding as B
    calls = [("GEMV", 1, 2048, 16384), ("SKINNY", 50, 1000, 4096), ("GEMV", 4, 4688, 32768),
             ("GEMV", 2, 100, 20480), ("SKINNY", 9, 520, 16384)]
    need = max(B.workspace_bytes(m, n, k, bits=8) for _, m, n, k in calls)
    need = max(need, B.workspace_bytes(1, 2048, 16384))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for i, (path, m, n, k) in enumerate(calls):
        say(f"int8 shared workspace call {i}: path={path} m={m} n={n} k={k}")
        w, x, b = exact_case8(m, n, k, seed=70 + i, dtype=torch.bfloat16, with_bias=(i % 2 == 0))
        packed, q, s = prepare8(w, dev)
        bd = b.to(dev) if b is not None else None
        y = run8(x.to(dev), packed, n, bd, path, workspace=ws)
        assert int(ws[:1 << 20].count_nonzero()) == 0, f"call {i}: exchange-slot header not left zero"
        y2 = run8(x.to(dev), packed, n, bd, path, workspace=ws)
        assert torch.equal(y, y2), f"call {i}: not deterministic"
        want = to_rne16(oracle.linear(bits(x), tag(torch.bfloat16), q, s, bits(b) if b is not None else None),
                        torch.bfloat16)
        bad = np.argwhere(y.cpu().to(torch.float64).numpy() != want)
        assert bad.size == 0, f"call {i} ({path} {m}x{n}x{k}): {len(bad)} mismatches"


W8_WORKLOADS = ["c1_m1_k1024_n1024", "c2_down_m50_k4096_n1024", "c3_gate_up_m1_k2048_n32768",
                "c3_down_m1_k16384_n2048", "c5_m1_k16384_n2048", "c4_m1024_k2048_n2560",
                "c4_m1024_k2048_n32768", "c4_m1024_k16384_n2048"]


@pytest.mark.parametrize("name", W8_WORKLOADS)
def test_int8_workload_shapes(dev, name):
    c = synth.case_by_name(name)
    say(f"int8 workload case {name}: m={c.m} k={c.k} n={c.n} {c.dtype} bias={c.bias}")
    packed, q, s = prepare8(synth.make_weight(c), dev)
    x = synth.make_x(c)
    b = synth.make_bias(c)
    y = run8(x.to(dev), packed, c.n, b.to(dev) if b is not None else None).cpu().to(torch.float64).numpy()
    xb, bb = bits(x), (bits(b) if b is not None else None)
    xnorm = np.linalg.norm(x.to(torch.float64).numpy(), axis=1)
    wmax = row_max_dequant(q, s)
    rng = np.random.default_rng(9)
    rows = np.concatenate([rng.integers(0, c.m, 4096), [0, c.m - 1, c.m - 1, 0]])
    cols = np.concatenate([rng.integers(0, c.n, 4096), [0, c.n - 1, 0, c.n - 1]])
    y_ref = oracle.linear_entries(xb, tag(c.torch_dtype), q, s, bb, rows, cols)
    check_close(y[rows, cols], y_ref, xnorm[rows], wmax[cols], f"int8 {name}")
