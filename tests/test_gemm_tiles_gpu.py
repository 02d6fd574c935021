"""Every tiling of the large-M path, bit for bit.

Each shape of tests/gemm_tilings.py reaches one (tile, waves, K split) of
the GEMM planner (checked on the host in test_boundary.py) with ragged M, N
and K.  Exact arithmetic (codes times 2^-3, small integer activations and
bias) makes every partial sum exact in FP32 in any order, so the GPU output
must equal the correctly rounded exact result on whole rows and columns at
tile edges; unsplit eight-wave tiles are also run with a row stride that is
not a multiple of 8, which takes the element-store epilogue instead of the
LDS-staged one.  The stream-K cuts of the same file likewise, each called
twice on one workspace.  INT4 and INT8 weights, bf16 and fp16."""
import numpy as np
import pytest
import torch

import oracle
from tests.gemm_tilings import STREAMK_TILINGS, TILINGS, streamk_id, tiling_id
from tests.gpu_util import bits as bits16
from tests.gpu_util import require_gpu, say, tag, to_rne16
from tests.test_linear_gpu import exact_case
from tests.test_w8_gpu import exact_case8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def edges(m, n, tm, tn):
    rows = sorted({0, 15, 16, tm - 1, tm, 2 * tm - 1, m - 2, m - 1} & set(range(m)))
    cols = sorted({0, 15, 16, tn - 1, tn, n - 17, n - 1} & set(range(n)))
    r = np.concatenate([np.repeat(rows, n), np.tile(np.arange(m), len(cols))])
    c = np.concatenate([np.tile(np.arange(n), len(rows)), np.repeat(cols, m)])
    return r, c


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("t", TILINGS, ids=tiling_id)
def test_tiling_bit_exact(dev, t, dtype):
    nbits, waves, tm, tn, split, (m, n, k) = t
    say(f"gemm tiling {tiling_id(t)} {dtype}")
    check_tiling(dev, nbits, "GEMM", tm, tn, m, n, k, dtype, row_strides=waves == 8 and not split)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("t", STREAMK_TILINGS, ids=streamk_id)
def test_streamk_bit_exact(dev, t, dtype):
    """Stream-K cuts (runs inside tiles, runs crossing tile ends) against the
    exact result, twice in a row on one workspace (the tile counters left
    zero by the first call), bit for bit the same both times; the
    LDS-staged and element-store epilogues."""
    nbits, tm, tn, inside, (m, n, k) = t
    say(f"stream-K tiling {streamk_id(t)} {dtype}")
    check_tiling(dev, nbits, "GEMM_STREAMK", tm, tn, m, n, k, dtype, row_strides=True, repeat=True)


def check_tiling(dev, nbits, path, tm, tn, m, n, k, dtype, row_strides, repeat=False):
    import weight_only_int4_rtn_amd as w4
    from weight_only_int4_rtn_amd import _binding as B
    make = exact_case8 if nbits == 8 else exact_case
    w, x, b = make(m, n, k, seed=m + 3 * n + 7 * k + nbits, dtype=dtype, with_bias=True)
    wd = w.to(dev)
    if nbits == 8:
        codes, scales = w4.quantize_int8(wd)
        packed = w4.pack_int8(codes, scales)
        q, s = oracle.quantize_int8(w.numpy())
    else:
        codes, scales = w4.quantize(wd)
        packed = w4.pack(codes, scales)
        q, s = oracle.quantize(w.numpy())
    xd, bd = x.to(dev), b.to(dev)
    rows, cols = edges(m, n, tm, tn)
    want = to_rne16(oracle.linear_entries(bits16(x), tag(dtype), q, s, bits16(b), rows, cols), dtype)
    need = max(w4.workspace_bytes(m, n, k, bits=nbits), w4.explain(m, n, k, path=w4.Path[path], bits=nbits)["workspace_bytes"])
    ws = torch.zeros(max(16, need), dtype=torch.uint8, device=dev)
    lds = [n] + ([n + 1] if row_strides else [])
    first = None
    for ldy in lds:
        for rep in range(2 if repeat else 1):
            ybuf = torch.full((m, ldy), -12352.0, dtype=dtype, device=dev)
            fn = B.lib().w8a16_linear if nbits == 8 else B.lib().w4a16_linear_act
            st = fn(0, int(w4.Path[path]), B._ptr(xd), B._act_tag(dtype), m, k, k, B._ptr(packed), n, B._ptr(bd),
                    B._ptr(ybuf), ldy, B._ptr(ws), ws.numel(), B._stream(dev))
            torch.cuda.synchronize()
            assert st == 0, B.status_string(st)
            assert int(ws[:1 << 20].count_nonzero()) == 0, "header counters not left zero"
            y = ybuf.cpu().to(torch.float64).numpy()
            got = y[rows, cols]
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, (f"ldy={ldy} call {rep}: {bad.size} mismatches, first at row {rows[bad[0]]} "
                                   f"col {cols[bad[0]]}: got {got[bad[0]]} want {want[bad[0]]}")
            if ldy > n:
                assert bool((ybuf[:, n:] == -12352.0).all()), "padding past n was written"
            if ldy == n:
                if first is None:
                    first = ybuf.clone()
                else:
                    assert torch.equal(ybuf, first), "repeated call differs"
