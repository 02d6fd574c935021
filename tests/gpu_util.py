"""Helpers shared by the GPU parity tests.

The reference values all come from the CPU oracle (``oracle/``) on the same
seeded inputs; nothing here is computed by the HIP library.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# Output tolerance, per element (m, n):
#   |y - y_ref| <= 1e-2 * ||x_m||_2 * max_k |W^[n, k]|
# and over a whole case  sum|y - y_ref| / sum|y_ref| <= 5e-3.
ABS_COEF = 1e-2
MEAN_REL = 5e-3


def require_gpu():
    """GPU tests fail (they are not skipped) when the GPU or library is missing."""
    assert torch.cuda.is_available(), "no GPU visible: GPU tests must run on an MI355X"
    import weight_only_int4_rtn_amd as w4
    w4.lib()
    return torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def tag(dtype) -> int:
    return oracle.BF16 if dtype == torch.bfloat16 else oracle.F16


def row_max_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """max_k |q[n,k] * s[n, k/128]| per output column n (exact in float64)."""
    n, k = q.shape
    g = np.abs(q.reshape(n, k // 128, 128)).max(axis=2).astype(np.float64)
    return (g * s.astype(np.float64)).max(axis=1)


def check_close(y_gpu: np.ndarray, y_ref: np.ndarray, xnorm: np.ndarray, wmax: np.ndarray, what: str):
    """Elementwise and mean-relative tolerance.  Arrays of equal shape; xnorm
    and wmax broadcast against them."""
    y_gpu = y_gpu.astype(np.float64)
    d = np.abs(y_gpu - y_ref)
    tau = ABS_COEF * xnorm * wmax
    bad = d > tau
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs beyond tolerance; first {idx.tolist()}: "
                             f"gpu {y_gpu[bad][:5]} ref {y_ref[bad][:5]} tol {np.broadcast_to(tau, d.shape)[bad][:5]}")
    denom = np.abs(y_ref).sum()
    if denom > 0:
        mre = d.sum() / denom
        assert mre <= MEAN_REL, f"{what}: mean relative error {mre:.3e} > {MEAN_REL}"
        return float(mre), float((d / np.maximum(tau, 1e-300)).max())
    assert d.max() == 0.0, f"{what}: nonzero output where the reference is exactly zero"
    return 0.0, 0.0


def to_rne16(y: np.ndarray, dtype) -> np.ndarray:
    """Round exact (float32-representable) values to the 16-bit dtype, as float64."""
    return torch.from_numpy(y.astype(np.float32)).to(dtype).to(torch.float64).numpy()
