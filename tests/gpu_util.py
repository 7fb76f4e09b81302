"""Helpers for the GPU parity tests: storage arrays to device tensors, the
tolerance measure, and the chained decode step through the C ABI."""

from __future__ import annotations

import sys

import numpy as np
import torch

from synth import configs as cf

# Normwise relative error bars per storage dtype: max|gpu - ref| / max|ref|.
TOL = {cf.F32: 1e-3, cf.BF16: 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    """Storage array (float32 or bf16 bits as uint16) -> device tensor of that dtype."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    if x.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    if x.dtype == np.int32:
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    raise TypeError(x.dtype)


def host_values(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact float64 values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(gpu: np.ndarray, ref: np.ndarray) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    denom = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (denom if denom > 0 else 1.0))


def assert_close(gpu, ref, dtype: str, what: str, tol: float | None = None):
    err = normwise(gpu, ref)
    bar = TOL[dtype] if tol is None else tol
    say(f"    {what}: normwise rel err {err:.3e} (bar {bar:.0e})")
    assert err <= bar, f"{what}: {err} > {bar}"


def bitwise_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Equal bit patterns, except that +0 and -0 compare equal."""
    x = a.detach().contiguous().view(torch.int32 if a.element_size() == 4 else torch.int16)
    y = b.detach().contiguous().view(torch.int32 if b.element_size() == 4 else torch.int16)
    zero = (a == 0) & (b == 0)
    return bool(((x == y) | zero).all().item())
