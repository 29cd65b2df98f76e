"""The allocation-free gradient preparation (static device scratch) against
the workspace entry point, through the C ABI."""

import math

import numpy as np
import pytest
import torch

from bwd_adamw_amd import lora as L
from bwd_adamw_amd import workloads as WL

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(g, n_pred, max_norm):
    """(norm, d_scale, d_stats) from each entry point on the same gradient."""
    out = []
    for noalloc in (False, True):
        d_scale = torch.full((1,), float("nan"), device=DEV)
        stats = torch.full((2,), float("nan"), device=DEV, dtype=torch.float64)
        if noalloc:
            norm = L.lora_grad_prepare_noalloc(g, n_pred, max_norm, d_scale, stats)
        else:
            ws = torch.empty(L.lora_grad_prepare_workspace_bytes(g.numel()), device=DEV,
                             dtype=torch.uint8)
            norm = L.lora_grad_prepare(g, n_pred, max_norm, d_scale, stats, True, ws)
        torch.cuda.synchronize()
        out.append((norm, d_scale.clone(), stats.clone()))
    return out


def test_noalloc_prepare_equals_the_workspace_entry_point_on_two_calls():
    """Two calls in a row, the second on a smaller arena (so fewer partials
    than the first call left in the scratch): each bitwise equal to
    lora_grad_prepare with a caller workspace."""
    for n, scale, max_norm, n_pred in ((5_000_001, 0.5, 2.0, 8), (1003, 10.0, 1.0, 4)):
        print("noalloc prepare", n, flush=True)
        g = WL.draw((n,), (510, 0, 0, 0, n % 97, "dY"), "normal", scale, DEV)
        (n0, s0, t0), (n1, s1, t1) = _both(g, n_pred, max_norm)
        assert n1 == n0 and math.isfinite(n1)
        assert torch.equal(s1, s0) and torch.equal(t1, t0)
        # and the prepared gradient's norm is max_norm when clipped
        if t1[1].item() < 1.0:
            assert np.linalg.norm(g.double().cpu().numpy() * s1.item()) == pytest.approx(
                max_norm, rel=1e-6)


def test_noalloc_prepare_vetoes_non_finite_then_recovers():
    """A veto (NaN scale, LORA_E_NONFINITE), then a finite call on the same
    scratch: the flags of the first call do not leak into the second."""
    g = WL.draw((70000,), (511, 0, 0, 0, 1, "dY"), "normal", 1.0, DEV)
    bad = g.clone()
    bad[777] = float("inf")
    d_scale = torch.zeros(1, device=DEV)
    with pytest.raises(L.LoraError) as e:
        L.lora_grad_prepare_noalloc(bad, 4, 1.0, d_scale, None)
    assert e.value.status == L.LORA_E_NONFINITE and math.isnan(d_scale.item())
    (n0, s0, t0), (n1, s1, t1) = _both(g[:4096], 4, 1.0)
    assert n1 == n0 and torch.equal(s1, s0) and torch.equal(t1, t0)


def test_noalloc_prepare_validates_before_work():
    g = torch.zeros(16, device=DEV)
    d_scale = torch.full((1,), 3.0, device=DEV)
    with pytest.raises(L.LoraError):
        L.lora_grad_prepare_noalloc(g, 0, 1.0, d_scale)
    with pytest.raises(L.LoraError):
        L.lora_grad_prepare_noalloc(g, 4, -1.0, d_scale)
    assert d_scale.item() == 3.0
