"""GPU linear layer with a fused input activation against the CPU oracle.

y = act(x) . dequant(Wq, s)^T + bias, act = SwiGLU over [up | gate] rows or
tanh-GELU ("Piper Kernels", section "ConvRot INT8").  The oracle evaluates the
activation in double and rounds it once to the activation dtype; the kernels
evaluate it in FP32 and round once, so an activated value may differ by one
16-bit unit where the FP32 result sits next to a rounding boundary.  Outputs
are compared with the layer's tolerance (tests/gpu_util.py), taking the norm
of the activated row as ||x_m||.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import bits, check_close, require_gpu, row_max_dequant, say, tag

pytestmark = pytest.mark.gpu

PATHS = ["GEMV", "MGEMV", "SKINNY", "GEMM", "AUTO"]
ACTS = {"swiglu": oracle.ACT_SWIGLU, "gelu": oracle.ACT_GELU_TANH}


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def w4():
    import weight_only_int4_rtn_amd as m
    return m


def make_case(m, n, k, seed, dtype, act, with_bias):
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(n, k, generator=g) * 0.02
    width = 2 * k if act == "swiglu" else k
    x = (torch.randn(m, width, generator=g) * 2.0).to(dtype)
    b = (torch.randn(n, generator=g) * 0.01).to(dtype) if with_bias else None
    return w, x, b


def reference(x, dtype, act, q, s, b):
    xb = bits(x)
    a = oracle.activate(xb, tag(dtype), ACTS[act])
    y = oracle.linear(a, tag(dtype), q, s, bits(b) if b is not None else None)
    at = torch.from_numpy(a.view(np.int16)).view(dtype).to(torch.float64).numpy()
    return y, np.linalg.norm(at, axis=1)


SHAPES = [(1, 48, 256), (3, 1000, 1024), (2, 72, 6144), (6, 200, 640), (16, 264, 2048), (50, 1024, 4096),
          (130, 100, 1152), (300, 520, 512)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("act", list(ACTS))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("m,n,k", SHAPES, ids=[f"m{m}_n{n}_k{k}" for m, n, k in SHAPES])
def test_fused_activation_within_tolerance(dev, path, act, dtype, m, n, k):
    lib = w4()
    w, x, b = make_case(m, n, k, seed=7 * m + n + k, dtype=dtype, act=act, with_bias=(n % 2 == 0))
    say(f"fused activation case path={path} act={act} dtype={dtype} m={m} n={n} k={k}")
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    q, s = oracle.quantize(w.numpy())
    y = lib.linear(x.to(dev), packed, n, b.to(dev) if b is not None else None, path=lib.Path[path],
                   act=lib.Act[act.upper() if act == "swiglu" else "GELU_TANH"])
    torch.cuda.synchronize()
    y_ref, anorm = reference(x, dtype, act, q, s, b)
    check_close(y.cpu().to(torch.float64).numpy(), y_ref, anorm[:, None], row_max_dequant(q, s)[None, :],
                f"{path} {act} m={m} n={n} k={k}")


def test_row_stride_and_deterministic(dev):
    """SwiGLU rows in a wider buffer (ldx > 2k), through the C ABI; two runs
    give identical bits."""
    from weight_only_int4_rtn_amd import _binding as B
    lib = w4()
    m, n, k = 5, 96, 1024
    w, x, _ = make_case(m, n, k, seed=3, dtype=torch.bfloat16, act="swiglu", with_bias=False)
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    q, s = oracle.quantize(w.numpy())
    ldx = 2 * k + 64
    xbuf = torch.zeros(m, ldx, dtype=torch.bfloat16)
    xbuf[:, :2 * k] = x
    xd = xbuf.to(dev)
    for path in ("MGEMV", "SKINNY", "GEMM"):
        need = B.workspace_bytes(m, n, k, B.Act.SWIGLU)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
        outs = []
        for _ in range(2):
            y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            st = B.lib().w4a16_linear_act(int(B.Act.SWIGLU), int(B.Path[path]), B._ptr(xd), B.BF16, m, k, ldx,
                                          B._ptr(packed), n, None, B._ptr(y), n, B._ptr(ws), ws.numel(),
                                          B._stream(dev))
            torch.cuda.synchronize()
            assert st == 0, B.status_string(st)
            outs.append(y.cpu())
        assert torch.equal(outs[0], outs[1]), path
        y_ref, anorm = reference(x, torch.bfloat16, "swiglu", q, s, None)
        check_close(outs[0].to(torch.float64).numpy(), y_ref, anorm[:, None], row_max_dequant(q, s)[None, :],
                    f"strided {path}")


def test_gemm_activation_leaves_slot_header_zero(dev):
    """A GEMM-path call with a materialised activation whose GEMM needs no
    K split (so no workspace of its own) keeps the activated input out of the
    exchange-slot header: the header stays zero, and a small-M call that
    finishes its K split through the slots, sharing the workspace, stays
    exact."""
    from tests.gpu_util import to_rne16
    lib = w4()
    g = torch.Generator().manual_seed(99)
    m, n, k = 300, 4104, 640
    w = torch.randn(n, k, generator=g) * 0.02
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    ws = torch.zeros(max(lib.workspace_bytes(m, n, k, lib.Act.GELU_TANH), lib.workspace_bytes(1, 2048, 16384)),
                     dtype=torch.uint8, device=dev)
    say(f"gemm activation workspace: m={m} n={n} k={k}")
    y = lib.linear(x.to(dev), packed, n, path=lib.Path.GEMM, act=lib.Act.GELU_TANH, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:1 << 20].count_nonzero()) == 0, "activated input written into the slot header"
    q, s = oracle.quantize(w.numpy())
    y_ref, anorm = reference(x, torch.bfloat16, "gelu", q, s, None)
    check_close(y.cpu().to(torch.float64).numpy(), y_ref, anorm[:, None], row_max_dequant(q, s)[None, :],
                "gemm gelu unsplit")
    # exact-arithmetic GEMV with a four-part split through the slots
    rng = np.random.default_rng(5)
    qi = rng.integers(-7, 8, size=(2048, 16384), dtype=np.int8)
    qi[:, ::128] = 7
    w2 = torch.from_numpy((qi * 2.0 ** -3).astype(np.float32))
    x2 = torch.from_numpy(rng.integers(-4, 5, size=(1, 16384)).astype(np.float32)).to(torch.bfloat16)
    c2, s2 = lib.quantize(w2.to(dev))
    y2 = lib.linear(x2.to(dev), lib.pack(c2, s2), 2048, path=lib.Path.GEMV, workspace=ws)
    torch.cuda.synchronize()
    q2, s2o = oracle.quantize(w2.numpy())
    want = to_rne16(oracle.linear(bits(x2), tag(torch.bfloat16), q2, s2o), torch.bfloat16)
    assert np.array_equal(y2.cpu().to(torch.float64).numpy(), want)
    assert int(ws[:1 << 20].count_nonzero()) == 0


FFN_CASES = [("swiglu", 1, 2048, 2048, torch.bfloat16), ("swiglu", 4, 1024, 1536, torch.bfloat16),
             ("gelu", 50, 1024, 4096, torch.bfloat16), ("gelu", 256, 512, 1024, torch.float16)]


@pytest.mark.parametrize("act,m,h,inter,dtype", FFN_CASES,
                         ids=[f"{a}_m{m}_h{h}_i{i}" for a, m, h, i, _ in FFN_CASES])
def test_ffn_composition(dev, act, m, h, inter, dtype):
    """An FFN block: up (or [up | gate]) projection, then the down projection
    with the activation fused into its input, against the oracle's
    composition (its up projection rounded to the activation dtype)."""
    lib = w4()
    g = torch.Generator().manual_seed(m + h + inter)
    width = 2 * inter if act == "swiglu" else inter
    w_up = torch.randn(width, h, generator=g) * 0.02
    w_dn = torch.randn(h, inter, generator=g) * 0.02
    b_dn = (torch.randn(h, generator=g) * 0.01).to(dtype)
    x = torch.randn(m, h, generator=g).to(dtype)
    say(f"ffn case act={act} m={m} hidden={h} intermediate={inter} dtype={dtype}")
    packs = []
    for w in (w_up, w_dn):
        c, sc = lib.quantize(w.to(dev))
        packs.append(lib.pack(c, sc))
    u = lib.linear(x.to(dev), packs[0], width)
    y = lib.linear(u, packs[1], h, b_dn.to(dev), act=lib.Act.SWIGLU if act == "swiglu" else lib.Act.GELU_TANH)
    torch.cuda.synchronize()
    q_up, s_up = oracle.quantize(w_up.numpy())
    q_dn, s_dn = oracle.quantize(w_dn.numpy())
    u_ref = torch.from_numpy(oracle.linear(bits(x), tag(dtype), q_up, s_up).astype(np.float32)).to(dtype)
    y_ref, anorm = reference(u_ref, dtype, act, q_dn, s_dn, b_dn)
    check_close(y.cpu().to(torch.float64).numpy(), y_ref, anorm[:, None], row_max_dequant(q_dn, s_dn)[None, :],
                f"ffn {act} m={m}")
