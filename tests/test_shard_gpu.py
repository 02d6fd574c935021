"""Shards of a packed weight (no requantization) against the oracle.

A shard of rows [start, start + length) (any start) or of group-aligned
columns must unpack to exactly those rows / columns of the oracle's canonical
codes and FP32 scales, give the oracle's linear layer on them, and fill the
padding rows of its last 16-row tile with code 0 and scale 0.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import bits, require_gpu, say, tag, to_rne16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def w4():
    import weight_only_int4_rtn_amd as m
    return m


def weights(n, k, seed):
    rng = np.random.default_rng(seed)
    qi = rng.integers(-7, 8, size=(n, k), dtype=np.int8)
    qi[:, ::128] = 7 * np.where(rng.random((n, k // 128)) < 0.5, 1, -1)
    return torch.from_numpy((qi * 2.0 ** -3).astype(np.float32))


def padding_ok(packed_bytes: np.ndarray, rows: int, k: int) -> bool:
    """Rows past `rows` in the last tile: every lane run 0x88.., scale 0."""
    tiles, groups = -(-rows // 16), k // 128
    pad = range(rows - (tiles - 1) * 16, 16)
    codes = packed_bytes[:tiles * groups * 1024].reshape(tiles, groups, 64, 16)
    scales = packed_bytes[tiles * groups * 1024:].view(np.float32).reshape(tiles, groups, 16)
    for r in pad:
        lanes = [r + 16 * q for q in range(4)]
        if not np.all(codes[tiles - 1][:, lanes, :] == 0x88) or not np.all(scales[tiles - 1][:, r] == 0):
            return False
    return True


CASES = [(100, 640, 0, 0, 100), (100, 640, 0, 17, 50), (100, 640, 0, 99, 1), (2048, 4096, 0, 1000, 700),
         (100, 640, 1, 128, 384), (100, 640, 1, 0, 640), (2048, 4096, 1, 2048, 128), (37, 1024, 1, 512, 512)]


@pytest.mark.parametrize("n,k,dim,start,length", CASES, ids=[f"n{a}_k{b}_d{c}_s{d}_l{e}" for a, b, c, d, e in CASES])
def test_shard_matches_oracle_slice(dev, n, k, dim, start, length):
    lib = w4()
    say(f"shard n={n} k={k} dim={dim} start={start} length={length}")
    w = weights(n, k, seed=n + k + start)
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    part = lib.shard(packed, n, k, dim, start, length)
    torch.cuda.synchronize()
    q, s = oracle.quantize(w.numpy())
    if dim == 0:
        qs, ss, rows, cols = q[start:start + length], s[start:start + length], length, k
    else:
        qs, ss, rows, cols = q[:, start:start + length], s[:, start // 128:(start + length) // 128], n, length
    assert part.numel() == lib.packed_bytes(rows, cols)
    c2, s2 = lib.unpack(part, rows, cols)
    assert np.array_equal(c2.cpu().numpy(), oracle.codes_to_nibbles(qs))
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), np.ascontiguousarray(ss).view(np.uint32))
    assert padding_ok(part.cpu().numpy(), rows, cols)
    # the shard computes the oracle's layer on those rows / columns, bit for bit
    # (exact arithmetic: codes * 2^-3 and small integer activations)
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.integers(-4, 5, size=(3, cols)).astype(np.float32)).to(torch.bfloat16)
    y = lib.linear(x.to(dev), part, rows)
    torch.cuda.synchronize()
    want = to_rne16(oracle.linear(bits(x), tag(torch.bfloat16), np.ascontiguousarray(qs), np.ascontiguousarray(ss)),
                    torch.bfloat16)
    assert np.array_equal(y.cpu().to(torch.float64).numpy(), want)


def test_row_shards_reassemble(dev):
    """Row shards of every size cover the weight: their outputs concatenate
    to the full layer's outputs exactly (column-parallel sharding)."""
    lib = w4()
    n, k = 300, 1024
    w = weights(n, k, seed=9)
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.integers(-4, 5, size=(5, k)).astype(np.float32)).to(torch.bfloat16).to(dev)
    full = lib.linear(x, packed, n)
    cuts = [0, 13, 16, 64, 150, 299, 300]
    parts = [lib.linear(x, lib.shard(packed, n, k, 0, a, b - a), b - a) for a, b in zip(cuts[:-1], cuts[1:])]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, dim=1), full)


def test_input_feature_shards_sum(dev):
    """Row-parallel emulation on one device: the layer on group-aligned input
    feature shards (the matching x columns each), partial outputs summed in
    FP32 and the bias added once, equals the unsharded layer within the
    layer's tolerance (the oracle's outputs as the reference)."""
    from tests.gpu_util import check_close, row_max_dequant
    lib = w4()
    m, n, k = 4, 264, 2048
    g = torch.Generator().manual_seed(3)
    w = torch.randn(n, k, generator=g) * 0.02
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    b = (torch.randn(n, generator=g) * 0.01).to(torch.bfloat16)
    codes, scales = lib.quantize(w.to(dev))
    packed = lib.pack(codes, scales)
    xd = x.to(dev)
    total = torch.zeros(m, n, dtype=torch.float32, device=dev)
    for start in range(0, k, 512):
        part = lib.shard(packed, n, k, 1, start, 512)
        total += lib.linear(xd[:, start:start + 512].contiguous(), part, n).float()
    y = (total + b.to(dev).float()).to(torch.bfloat16)
    torch.cuda.synchronize()
    q, s = oracle.quantize(w.numpy())
    y_ref = oracle.linear(bits(x), tag(torch.bfloat16), q, s, bits(b))
    xnorm = np.linalg.norm(x.to(torch.float64).numpy(), axis=1)[:, None]
    check_close(y.cpu().to(torch.float64).numpy(), y_ref, xnorm, row_max_dequant(q, s)[None, :], "K shards summed")


# --- INT8 weights --------------------------------------------------------------


def weights8(n, k, seed):
    rng = np.random.default_rng(seed)
    qi = rng.integers(-127, 128, size=(n, k)).astype(np.int16)
    qi[:, ::128] = 127 * np.where(rng.random((n, k // 128)) < 0.5, 1, -1)
    return torch.from_numpy((qi * 2.0 ** -3).astype(np.float32))


def padding8_ok(packed_bytes: np.ndarray, rows: int, k: int) -> bool:
    """INT8: rows past `rows` in the last tile: both halves' lane runs 0x80.., scale 0."""
    tiles, groups = -(-rows // 16), k // 128
    pad = range(rows - (tiles - 1) * 16, 16)
    codes = packed_bytes[:tiles * groups * 2048].reshape(tiles, groups, 2, 64, 16)
    scales = packed_bytes[tiles * groups * 2048:].view(np.float32).reshape(tiles, groups, 16)
    for r in pad:
        lanes = [r + 16 * q for q in range(4)]
        if not np.all(codes[tiles - 1][:, :, lanes, :] == 0x80) or not np.all(scales[tiles - 1][:, r] == 0):
            return False
    return True


@pytest.mark.parametrize("n,k,dim,start,length", CASES, ids=[f"n{a}_k{b}_d{c}_s{d}_l{e}" for a, b, c, d, e in CASES])
def test_int8_shard_matches_oracle_slice(dev, n, k, dim, start, length):
    lib = w4()
    say(f"int8 shard n={n} k={k} dim={dim} start={start} length={length}")
    w = weights8(n, k, seed=n + k + start + 1)
    codes, scales = lib.quantize_int8(w.to(dev))
    packed = lib.pack_int8(codes, scales)
    part = lib.shard(packed, n, k, dim, start, length, bits=8)
    torch.cuda.synchronize()
    q, s = oracle.quantize_int8(w.numpy())
    if dim == 0:
        qs, ss, rows, cols = q[start:start + length], s[start:start + length], length, k
    else:
        qs, ss, rows, cols = q[:, start:start + length], s[:, start // 128:(start + length) // 128], n, length
    assert part.numel() == lib.packed_bytes(rows, cols, bits=8)
    c2, s2 = lib.unpack_int8(part, rows, cols)
    assert np.array_equal(c2.cpu().numpy(), qs)
    assert np.array_equal(s2.cpu().numpy().view(np.uint32), np.ascontiguousarray(ss).view(np.uint32))
    assert padding8_ok(part.cpu().numpy(), rows, cols)
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.integers(-4, 5, size=(3, cols)).astype(np.float32)).to(torch.bfloat16)
    y = lib.linear(x.to(dev), part, rows, bits=8)
    torch.cuda.synchronize()
    want = to_rne16(oracle.linear(bits(x), tag(torch.bfloat16), np.ascontiguousarray(qs), np.ascontiguousarray(ss)),
                    torch.bfloat16)
    assert np.array_equal(y.cpu().to(torch.float64).numpy(), want)
