"""Shared test utilities: error metrics and tensor conversion (no method math)."""

import numpy as np
import torch


def np64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel_err(got, ref):
    """max|got - ref| / max|ref| over the whole tensor."""
    got, ref = np64(got), np64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.abs(ref).max()
    num = np.abs(got - ref).max()
    if den == 0:
        return float(num)
    return float(num / den)


def gpu_available():
    try:
        return torch.cuda.is_available()
    except Exception:
        return False
