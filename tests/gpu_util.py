"""Helpers for the GPU parity tests (marshalling only, no method arithmetic)."""
from __future__ import annotations

import sys

import numpy as np
import torch

LOSS_RTOL = 1e-4          # per-alpha loss, relative
GEMM_TOL = 2e-3           # W4A16 outputs: max |dY| <= GEMM_TOL * max |Y|


def dev_tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def say(*args):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print(*args, flush=True)
    sys.stdout.flush()


def gemm_tolerance(Yref: np.ndarray, out: str) -> np.ndarray:
    """Per-element bound on |Y - Yref| for the W4A16 product.

    float32 output: GEMM_TOL * max |Yref| everywhere.  bf16 output: plus the
    rounding of the element itself, at most 2^-8 (the unit roundoff of an
    8-bit significand) of its float32 value, which lies within the float32
    bound of Yref."""
    base = GEMM_TOL * np.abs(Yref).max()
    if out != "bf16":
        return np.full(Yref.shape, base)
    return base + 2.0 ** -8 * (np.abs(Yref) + base)


def tie_band(losses: np.ndarray, rtol: float = 2 * LOSS_RTOL):
    """Indices whose loss is within rtol of the minimum (near-tie band)."""
    m = losses.min()
    return [k for k in range(len(losses)) if losses[k] <= m * (1 + rtol)]
