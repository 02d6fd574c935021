"""In-place updates of a packed weight against the CPU oracle.

W' = beta * dequant(W) + alpha * U (a dense update, or a low-rank product
accumulated in FP32), requantized with nearest or seeded stochastic rounding
("Piper Kernels", sections "ConvRot INT8" and "Stochastic quantization").
Every step is specified as an FP32 operation, so codes and scales must equal
the oracle's byte for byte, in both rounding modes.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def w4():
    import weight_only_int4_rtn_amd as m
    return m


def oracle_arrays(t: torch.Tensor):
    """float32 arrays as they are; 16-bit tensors as raw bits plus their tag."""
    if t.dtype == torch.float32:
        return t.numpy(), None
    return t.contiguous().view(torch.int16).numpy().view(np.uint16), (oracle.BF16 if t.dtype == torch.bfloat16
                                                                       else oracle.F16)


def check(lib, packed, n, k, q_want, s_want, what):
    codes, scales = lib.unpack(packed, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), oracle.codes_to_nibbles(q_want)), f"{what}: codes differ"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_want.view(np.uint32)), f"{what}: scales differ"


DENSE = [(40, 640, torch.float32, 1.0, 1.0), (16, 128, torch.bfloat16, 0.5, 1.0), (100, 1024, torch.float16, -1.5, 0.75),
         (2048, 4096, torch.bfloat16, 0.25, 1.0)]


@pytest.mark.parametrize("seed", [None, 2024, (1 << 64) - 3], ids=["nearest", "seed2024", "seedbig"])
@pytest.mark.parametrize("n,k,dt,alpha,beta", DENSE, ids=[f"n{a}_k{b}_{str(c)[6:]}_a{d}_b{e}" for a, b, c, d, e in DENSE])
def test_dense_update(dev, n, k, dt, alpha, beta, seed):
    lib = w4()
    say(f"dense update n={n} k={k} dtype={dt} alpha={alpha} beta={beta} seed={seed}")
    g = torch.Generator().manual_seed(n + k)
    w = torch.randn(n, k, generator=g) * 0.02
    u = (torch.randn(n, k, generator=g) * 0.01).to(dt)
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    lib.update_(packed, n, k, update=u.to(dev), alpha=alpha, beta=beta, seed=seed)
    q, s = oracle.quantize(w.numpy())
    ua, tag = oracle_arrays(u)
    q2, s2 = oracle.update(q, s, upd=ua, alpha=alpha, beta=beta, seed=seed, dtype_tag=tag)
    check(lib, packed, n, k, q2, s2, f"dense n={n} seed={seed}")
    if seed is not None:
        assert not np.array_equal(q2, oracle.update(q, s, upd=ua, alpha=alpha, beta=beta, dtype_tag=tag)[0])


LOWRANK = [(48, 256, 1, torch.float32), (100, 640, 7, torch.bfloat16), (2048, 16384, 16, torch.bfloat16),
           (33, 1152, 4, torch.float16)]


@pytest.mark.parametrize("seed", [None, 99], ids=["nearest", "seed99"])
@pytest.mark.parametrize("n,k,rank,dt", LOWRANK, ids=[f"n{a}_k{b}_r{c}_{str(d)[6:]}" for a, b, c, d in LOWRANK])
def test_lowrank_update(dev, n, k, rank, dt, seed):
    lib = w4()
    say(f"low-rank update n={n} k={k} rank={rank} dtype={dt} seed={seed}")
    g = torch.Generator().manual_seed(n * 3 + k + rank)
    w = torch.randn(n, k, generator=g) * 0.02
    m1 = (torch.randn(n, rank, generator=g) * 0.05).to(dt)
    m2 = (torch.randn(rank, k, generator=g) * 0.05).to(dt)
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    lib.update_(packed, n, k, mat1=m1.to(dev), mat2=m2.to(dev), alpha=0.8, beta=1.0, seed=seed)
    q, s = oracle.quantize(w.numpy())
    a1, tag = oracle_arrays(m1)
    a2, _ = oracle_arrays(m2)
    q2, s2 = oracle.update(q, s, mat1=a1, mat2=a2, alpha=0.8, beta=1.0, seed=seed, dtype_tag=tag)
    check(lib, packed, n, k, q2, s2, f"low-rank n={n} rank={rank} seed={seed}")


def test_strided_update_and_repeatability(dev):
    """A dense update in a wider buffer (ldu > k) through the C ABI, and the
    same seeded update applied to two copies gives the same bytes."""
    from weight_only_int4_rtn_amd import _binding as B
    import ctypes
    lib = w4()
    n, k = 50, 384
    g = torch.Generator().manual_seed(5)
    w = torch.randn(n, k, generator=g) * 0.02
    u = torch.randn(n, k + 16, generator=g) * 0.01
    codes, scales = lib.quantize(w.to(dev))
    p1 = lib.pack(codes, scales)
    p2 = p1.clone()
    ud = u.to(dev)
    seed = ctypes.pointer(ctypes.c_uint64(31337))
    for p in (p1, p2):
        st = B.lib().w4a16_update_packed(B._ptr(p), n, k, B._ptr(ud), k + 16, None, None, 0, B.F32,
                                         ctypes.c_float(1.0), ctypes.c_float(1.0), seed, B._stream(dev))
        assert st == 0, B.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    q, s = oracle.quantize(w.numpy())
    q2, s2 = oracle.update(q, s, upd=np.ascontiguousarray(u.numpy()[:, :k]), seed=31337)
    check(lib, p1, n, k, q2, s2, "strided")


# --- INT8 weights --------------------------------------------------------------


def check8(lib, packed, n, k, q_want, s_want, what):
    codes, scales = lib.unpack_int8(packed, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), q_want), f"{what}: codes differ"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), s_want.view(np.uint32)), f"{what}: scales differ"


@pytest.mark.parametrize("seed", [None, 2024, (1 << 64) - 3], ids=["nearest", "seed2024", "seedbig"])
@pytest.mark.parametrize("n,k,dt,alpha,beta", DENSE, ids=[f"n{a}_k{b}_{str(c)[6:]}_a{d}_b{e}" for a, b, c, d, e in DENSE])
def test_int8_dense_update(dev, n, k, dt, alpha, beta, seed):
    lib = w4()
    say(f"int8 dense update n={n} k={k} dtype={dt} alpha={alpha} beta={beta} seed={seed}")
    g = torch.Generator().manual_seed(n + k + 1)
    w = torch.randn(n, k, generator=g) * 0.02
    u = (torch.randn(n, k, generator=g) * 0.001).to(dt)
    codes, scales = lib.quantize_int8(w.to(dev))
    packed = lib.pack_int8(codes, scales)
    lib.update_(packed, n, k, update=u.to(dev), alpha=alpha, beta=beta, seed=seed, bits=8)
    q, s = oracle.quantize_int8(w.numpy())
    ua, tag = oracle_arrays(u)
    q2, s2 = oracle.update(q, s, upd=ua, alpha=alpha, beta=beta, seed=seed, dtype_tag=tag, bits=8)
    check8(lib, packed, n, k, q2, s2, f"int8 dense n={n} seed={seed}")
    if seed is not None:
        assert not np.array_equal(q2, oracle.update(q, s, upd=ua, alpha=alpha, beta=beta, dtype_tag=tag, bits=8)[0])


@pytest.mark.parametrize("seed", [None, 99], ids=["nearest", "seed99"])
@pytest.mark.parametrize("n,k,rank,dt", LOWRANK, ids=[f"n{a}_k{b}_r{c}_{str(d)[6:]}" for a, b, c, d in LOWRANK])
def test_int8_lowrank_update(dev, n, k, rank, dt, seed):
    lib = w4()
    say(f"int8 low-rank update n={n} k={k} rank={rank} dtype={dt} seed={seed}")
    g = torch.Generator().manual_seed(n * 3 + k + rank + 1)
    w = torch.randn(n, k, generator=g) * 0.02
    m1 = (torch.randn(n, rank, generator=g) * 0.02).to(dt)
    m2 = (torch.randn(rank, k, generator=g) * 0.02).to(dt)
    codes, scales = lib.quantize_int8(w.to(dev))
    packed = lib.pack_int8(codes, scales)
    lib.update_(packed, n, k, mat1=m1.to(dev), mat2=m2.to(dev), alpha=0.8, beta=1.0, seed=seed, bits=8)
    q, s = oracle.quantize_int8(w.numpy())
    a1, tag = oracle_arrays(m1)
    a2, _ = oracle_arrays(m2)
    q2, s2 = oracle.update(q, s, mat1=a1, mat2=a2, alpha=0.8, beta=1.0, seed=seed, dtype_tag=tag, bits=8)
    check8(lib, packed, n, k, q2, s2, f"int8 low-rank n={n} rank={rank} seed={seed}")
