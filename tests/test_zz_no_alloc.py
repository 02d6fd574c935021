"""w4a16_linear_noalloc: the linear layer with its workspace in the
library's own fixed scratch array (for callers that cannot allocate).  Its
results equal w4a16_linear's (explicit workspace) bit for bit, call after
call on the same array, each call on a smaller input than the one before;
a call whose plan needs more than the array holds is refused before any
launch."""
import pytest
import torch

from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

# (m, n, k, dtype), each smaller than the one before: GEMV with a K split
# finished through the exchange slots (the scratch header), SKINNY with
# partial sums and the reduce kernel, MGEMV split through the slots, GEMV
# unsplit
CALLS = [(50, 1000, 4096, torch.bfloat16), (1, 2048, 16384, torch.float16),
         (6, 520, 8192, torch.bfloat16), (1, 1040, 1024, torch.bfloat16)]


def _setup(dev, g, m, n, k, dtype):
    import weight_only_int4_rtn_amd as w4
    c, s = w4.quantize((torch.randn(n, k, generator=g) * 0.02).to(dev))
    x = torch.randn(m, k, generator=g).to(dtype).to(dev)
    b = (torch.randn(n, generator=g) * 0.01).to(dtype).to(dev)
    return x, w4.pack(c, s), b


def test_noalloc_equals_linear_call_after_call():
    dev = require_gpu()
    import weight_only_int4_rtn_amd as w4
    g = torch.Generator().manual_seed(21)
    for rep in range(2):
        for m, n, k, dtype in CALLS:
            say(f"rep {rep}: noalloc m={m} n={n} k={k} {dtype}")
            x, p, b = _setup(dev, g, m, n, k, dtype)
            ws = torch.zeros(max(16, w4.workspace_bytes(m, n, k)), dtype=torch.uint8, device=dev)
            ref = w4.linear(x, p, n, b, workspace=ws)
            y = torch.full((m, n), float("nan"), dtype=dtype, device=dev)
            w4.linear_noalloc(x, p, n, b, out=y)
            torch.cuda.synchronize()
            assert torch.equal(y, ref), f"rep {rep} m={m} n={n} k={k}"


def test_noalloc_refuses_plans_beyond_the_scratch():
    dev = require_gpu()
    import weight_only_int4_rtn_amd as w4
    # M = 1024, K = 16384, N = 2048 takes the GEMM with a K split whose FP32
    # partial sums need more than the scratch array holds
    m, n, k = 1024, 2048, 16384
    assert w4.explain(m, n, k)["workspace_bytes"] > w4._binding.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(m, k, dtype=torch.bfloat16, device=dev)
    p = torch.zeros(w4.packed_bytes(n, k), dtype=torch.uint8, device=dev)
    y = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError) as ei:
        w4.linear_noalloc(x, p, n, out=y)
    assert ei.value.status == 3  # W4A16_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a refused call launched something"
