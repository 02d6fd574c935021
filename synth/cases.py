"""The five seeded workloads (36 cases) and their input recipes.

Every tensor is drawn on the CPU with its own ``torch.Generator`` in float32
(``torch.randn``), so the same case always produces the same bits:

  weight  seed = 1000*config + shape_index            (shared across M)
  x       seed = 1000*config + 100 + case_index
  bias    seed = 1000*config + 200 + shape_index

Recipes per workload (sigma is a standard deviation):
  1  M=1, K=1024, N=1024; x bf16 N(0,1); W N(0,0.02); no bias.
  2  action-chunk MLP, M=50: up K=1024 N=4096 (no bias) and down K=4096
     N=1024 with a bf16 N(0,0.01) bias; each projection gets its own x.
  3  decode projections, M in {1,4,16}, W N(0,0.02) where each element is,
     independently with probability 0.01, replaced by a N(0,0.2) outlier:
     gate_up K=2048 N=32768, down K=16384 N=2048, qkv K=2048 N=2560,
     o K=2048 N=2048.
  4  prefill, M=1024, fp16 x and bias (bias N(0,0.01)): K=2048 N=2560,
     K=2048 N=32768, K=16384 N=2048.
  5  roofline sweep, M in {1,8,64,256,1024,4096} x (K,N) in
     {(1024,4096),(2048,16384),(16384,2048)}; x bf16 N(0,1) with every
     feature k % 64 == 0 multiplied by 10 (in fp32, before the one cast);
     W N(0,0.02) with row n's group (n mod K/128) set to zero.

x is cast from float32 to bf16/fp16 once, round-to-nearest-even (torch's
cast); W stays float32.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    config: int          # 1..5
    shape_index: int     # index of the (K, N) weight within its workload
    case_index: int      # index of the case within its workload
    m: int
    k: int
    n: int
    dtype: str           # "bf16" or "f16" (activation, bias and output dtype)
    bias: bool
    outliers: bool = False
    zero_group: bool = False
    hot_features: bool = False

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float16

    def alg_bytes(self) -> int:
        """Bytes the layer must move: packed codes, FP32 scales, x, y (and bias)."""
        b = self.n * self.k // 2 + 4 * self.n * (self.k // 128) + 2 * self.m * self.k + 2 * self.m * self.n
        return b + (2 * self.n if self.bias else 0)

    def flops(self) -> int:
        return 2 * self.m * self.n * self.k


def _build() -> list[Case]:
    cases: list[Case] = []
    # 1: single small linear
    cases.append(Case("c1_m1_k1024_n1024", 1, 0, 0, 1, 1024, 1024, "bf16", False))
    # 2: action-chunk MLP up and down
    cases.append(Case("c2_up_m50_k1024_n4096", 2, 0, 0, 50, 1024, 4096, "bf16", False))
    cases.append(Case("c2_down_m50_k4096_n1024", 2, 1, 1, 50, 4096, 1024, "bf16", True))
    # 3: decode projections with outliers
    shapes3 = [("gate_up", 2048, 32768), ("down", 16384, 2048), ("qkv", 2048, 2560), ("o", 2048, 2048)]
    ci = 0
    for m in (1, 4, 16):
        for si, (nm, k, n) in enumerate(shapes3):
            cases.append(Case(f"c3_{nm}_m{m}_k{k}_n{n}", 3, si, ci, m, k, n, "bf16", False, outliers=True))
            ci += 1
    # 4: prefill, fp16 with bias
    shapes4 = [(2048, 2560), (2048, 32768), (16384, 2048)]
    for si, (k, n) in enumerate(shapes4):
        cases.append(Case(f"c4_m1024_k{k}_n{n}", 4, si, si, 1024, k, n, "f16", True))
    # 5: sweep
    shapes5 = [(1024, 4096), (2048, 16384), (16384, 2048)]
    ci = 0
    for m in (1, 8, 64, 256, 1024, 4096):
        for si, (k, n) in enumerate(shapes5):
            cases.append(Case(f"c5_m{m}_k{k}_n{n}", 5, si, ci, m, k, n, "bf16", False,
                              zero_group=True, hot_features=True))
            ci += 1
    return cases


CONFIGS = _build()


def all_cases() -> list[Case]:
    return list(CONFIGS)


def case_by_name(name: str) -> Case:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def make_weight(c: Case) -> torch.Tensor:
    """float32 [N, K] weight of the case (CPU)."""
    g = _gen(1000 * c.config + c.shape_index)
    w = torch.randn(c.n, c.k, generator=g, dtype=torch.float32) * 0.02
    if c.outliers:
        mask = torch.rand(c.n, c.k, generator=g, dtype=torch.float32) < 0.01
        vals = torch.randn(c.n, c.k, generator=g, dtype=torch.float32) * 0.2
        w = torch.where(mask, vals, w)
    if c.zero_group:
        groups = c.k // 128
        rows = torch.arange(c.n)
        g_of_row = rows % groups
        cols = g_of_row[:, None] * 128 + torch.arange(128)[None, :]
        w[rows[:, None], cols] = 0.0
    return w


def make_x(c: Case) -> torch.Tensor:
    """[M, K] activations of the case, in its 16-bit dtype (CPU)."""
    g = _gen(1000 * c.config + 100 + c.case_index)
    x = torch.randn(c.m, c.k, generator=g, dtype=torch.float32)
    if c.hot_features:
        x[:, ::64] *= 10.0
    return x.to(c.torch_dtype)


def make_bias(c: Case):
    """[N] bias in the case's dtype, or None."""
    if not c.bias:
        return None
    g = _gen(1000 * c.config + 200 + c.shape_index)
    return (torch.randn(c.n, generator=g, dtype=torch.float32) * 0.01).to(c.torch_dtype)


def to_bits16(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bf16/fp16 CPU tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
