"""GPU quantization and packing against the CPU oracle: bit-exact.

Codes and scales are integer / exactly rounded results, so the GPU must
reproduce the oracle byte for byte (both take every rounding decision in
FP32: the scale division, the quotient and the ties-to-even rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bits, require_gpu, say

pytestmark = pytest.mark.gpu

WEIGHT_CASES = ["c1_m1_k1024_n1024", "c2_up_m50_k1024_n4096", "c2_down_m50_k4096_n1024",
                "c3_gate_up_m1_k2048_n32768", "c3_down_m1_k16384_n2048", "c3_qkv_m1_k2048_n2560",
                "c3_o_m1_k2048_n2048", "c4_m1024_k2048_n2560", "c4_m1024_k2048_n32768",
                "c4_m1024_k16384_n2048", "c5_m1_k1024_n4096", "c5_m1_k2048_n16384",
                "c5_m1_k16384_n2048"]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def gpu_quantize(w_cpu: torch.Tensor, dev):
    import weight_only_int4_rtn_amd as w4
    codes, scales = w4.quantize(w_cpu.to(dev))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def oracle_canonical(w_cpu: torch.Tensor, dtype_tag=None):
    if w_cpu.dtype == torch.float32:
        q, s = oracle.quantize(w_cpu.numpy())
    else:
        q, s = oracle.quantize(bits(w_cpu), dtype_tag)
    return oracle.codes_to_nibbles(q), s


@pytest.mark.parametrize("name", WEIGHT_CASES)
def test_quantize_matches_oracle_on_workload_weights(dev, name):
    c = synth.case_by_name(name)
    say(f"quantize parity: {name} n={c.n} k={c.k}")
    w = synth.make_weight(c)
    codes, scales = gpu_quantize(w, dev)
    want_codes, want_scales = oracle_canonical(w)
    assert np.array_equal(scales.view(np.uint32), want_scales.view(np.uint32)), "scales differ"
    diff = np.flatnonzero(codes != want_codes)
    assert diff.size == 0, f"{diff.size} code bytes differ, first at {diff[:5]}"


def edge_weights():
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((48, 1024)) * 0.02).astype(np.float32)
    # exact ties: max 7 gives scale 1, then x.5 values
    w[0, :128] = 0.0
    w[0, 0] = 7.0
    w[0, 1:12] = [0.5, 1.5, 2.5, 3.5, -2.5, -0.5, 6.5, 4.5, 5.5, -1.5, -3.5]
    w[1, 128:256] = 0.0                       # all-zero group
    w[2, 256:384] = -0.0                      # negative zeros
    w[3, :128] *= np.float32(1e-39)           # subnormal group
    w[4, 128:256] = 0.0
    w[4, 128] = np.float32(2.0 ** -149) * 2   # scale underflows to 0
    w[4, 129] = -np.float32(2.0 ** -149)
    w[5, 256:384] = 0.0
    w[5, 256] = np.float32(2.0 ** -149) * 4   # scale = smallest subnormal
    w[5, 257] = -np.float32(2.0 ** -149) * 3
    w[6, :] *= np.float32(1e30)               # huge magnitudes
    w[7, 384:512] = np.float32(0.7) * np.arange(128, dtype=np.float32) / np.float32(127.0)
    w[8, :] = np.float32(1.0)                 # constant rows
    w[9, ::2] = -w[9, 1::2]
    return w


def test_quantize_edge_cases(dev):
    w = torch.from_numpy(edge_weights())
    say("quantize parity: edge cases")
    codes, scales = gpu_quantize(w, dev)
    want_codes, want_scales = oracle_canonical(w)
    assert np.array_equal(scales.view(np.uint32), want_scales.view(np.uint32))
    assert np.array_equal(codes, want_codes)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_quantize_16bit_weights(dev, dtype):
    rng = np.random.default_rng(5)
    w = torch.from_numpy((rng.standard_normal((40, 640)) * 0.02).astype(np.float32)).to(dtype)
    say(f"quantize parity: {dtype} weights")
    codes, scales = gpu_quantize(w, dev)
    want_codes, want_scales = oracle_canonical(w, oracle.BF16 if dtype == torch.bfloat16 else oracle.F16)
    assert np.array_equal(scales.view(np.uint32), want_scales.view(np.uint32))
    assert np.array_equal(codes, want_codes)


def test_quantize_strided_rows(dev):
    import weight_only_int4_rtn_amd as w4
    rng = np.random.default_rng(8)
    full = torch.from_numpy((rng.standard_normal((24, 512)) * 0.02).astype(np.float32))
    view = full[:, :384]  # row stride 512, k = 384
    say("quantize parity: strided rows")
    codes, scales = w4.quantize(full.to(dev)[:, :384])
    torch.cuda.synchronize()
    want_codes, want_scales = oracle_canonical(view.contiguous())
    assert np.array_equal(scales.cpu().numpy(), want_scales)
    assert np.array_equal(codes.cpu().numpy(), want_codes)


def test_quantize_is_deterministic(dev):
    c = synth.case_by_name("c3_qkv_m1_k2048_n2560")
    w = synth.make_weight(c).to(dev)
    import weight_only_int4_rtn_amd as w4
    say("quantize determinism")
    a = w4.quantize(w)
    b = w4.quantize(w)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("n,k", [(16, 128), (17, 256), (1000, 384), (2056, 1152)])
def test_pack_roundtrip_any_nibbles(dev, n, k):
    """unpack(pack(codes, scales)) is the identity on arbitrary bytes (codes -8 included)."""
    import weight_only_int4_rtn_amd as w4
    rng = np.random.default_rng(n + k)
    codes = torch.from_numpy(rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)).to(dev)
    scales = torch.from_numpy(rng.standard_normal((n, k // 128)).astype(np.float32)).to(dev)
    say(f"pack round trip n={n} k={k}")
    packed = w4.pack(codes, scales)
    assert packed.numel() == w4.packed_bytes(n, k)
    c2, s2 = w4.unpack(packed, n, k)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes)
    assert torch.equal(s2.view(torch.int32), scales.view(torch.int32))
