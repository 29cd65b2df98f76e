"""The C-ABI library without a GPU: it loads, exports every symbol that
include/lora.h declares, rejects invalid arguments before touching a device,
and its host helpers agree with the oracle."""

import ctypes as C
import math
import os
import re

import numpy as np
import pytest
import torch

import oracle as O
from bwd_adamw_amd import lora as L

# The validation tests below pass placeholder pointers; they must only ever
# run where no GPU exists, so that a validation bug cannot launch a kernel.
no_device = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="placeholder-pointer tests run only on GPU-less hosts")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lora.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    declared = _declared()
    assert len(declared) >= 11
    assert sorted(L.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    assert L.lora_status_string(0) == "ok"
    assert "vetoed" in L.lora_status_string(-6)
    assert L.lora_status_string(12345) == "unknown status"


def test_scaling_matches_oracle():
    for alpha, r, mode in ((8, 4, "standard"), (16, 8, "standard"), (32, 32, "rslora"), (64, 64, "standard")):
        assert L.lora_scaling(alpha, r, mode == "rslora") == pytest.approx(O.scaling(alpha, r, mode), rel=1e-15)


@pytest.mark.parametrize("k", list(range(0, 12)) + [40, 55, 99, 100, 150])
def test_lr_schedule_matches_oracle(k):
    got = L.lora_lr_at(k, 1e-4, 1, 10, 100, 1e-6)
    ref = O.lr_at(k, 1e-4, "cosine", 10, 100, 1e-6)
    assert got == pytest.approx(ref, rel=1e-14, abs=1e-20)
    assert L.lora_lr_at(k, 3e-4, 0) == 3e-4


def _lin(**kw):
    d = dict(tokens=8, in_dim=16, out_dim=16, rank=4, w_dtype=L.F32, scale=2.0, W=256, A=256, B=256,
             dora_mag=None, dora_norm=None)
    d.update(kw)
    return L.LoraLinear(**d)


@no_device
@pytest.mark.parametrize("kw,status", [
    (dict(tokens=0), -2), (dict(in_dim=-4), -2), (dict(rank=0), -2), (dict(rank=132), -2),
    (dict(rank=32), -2), (dict(w_dtype=7), -3), (dict(in_dim=18), -4), (dict(rank=6), -4),
    (dict(W=None), -1), (dict(A=264), -4), (dict(dora_mag=256), -1),
    (dict(w_dtype=L.BF16, in_dim=20), -4),
    (dict(w_dtype=2, in_dim=48), -2), (dict(w_dtype=4, in_dim=288), -2),
    (dict(w_dtype=5, in_dim=1 << 23, out_dim=8), -2), (dict(w_dtype=6), -3),
])
def test_invalid_descriptor_is_rejected_before_any_launch(kw, status):
    lin = _lin(**kw)
    assert L.lib().lora_workspace_bytes(C.byref(lin)) == 0
    rc = L.lib().lora_forward(C.byref(lin), 256, 256, 256, None, None, 256, 1 << 20, None)
    assert rc == status


@no_device
def test_workspace_and_dropout_validation():
    lin = _lin(tokens=128, in_dim=2048, out_dim=2048, rank=8)   # needs split partials
    need = L.lib().lora_workspace_bytes(C.byref(lin))
    assert need > 1024
    assert L.lib().lora_forward(C.byref(lin), 256, 256, 256, None, None, 256, 16, None) == -5
    assert L.lib().lora_forward(C.byref(lin), 256, 256, 256, None, None, None, need, None) == -5
    bad = L.make_dropout(1, 0, 0, 0, 0, 1.0)
    assert L.lib().lora_forward(C.byref(lin), 256, 256, 256, None, C.byref(bad), 256, need, None) == -1
    nan = L.make_dropout(1, 0, 0, 0, 0, math.nan)
    assert L.lib().lora_dropout_mask(C.byref(nan), 4, 4, 256, None) == -1
    # backward: dMag without DoRA, misaligned outputs
    assert L.lib().lora_backward(C.byref(lin), 256, 256, 256, 256, 256, 256, 256, 256, 0, None,
                                 256, need, None) == -1
    assert L.lib().lora_backward(C.byref(lin), 256, 256, 256, None, 260, 256, 256, None, 0, None,
                                 256, need, None) == -4


@no_device
def test_optimizer_entry_validation():
    lib = L.lib()
    hp = L.LoraAdamwHparams(1e-4, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    seg = (L.LoraSegment * 1)(L.LoraSegment(0, 6, 0))
    assert lib.lora_adamw_step(256, 256, 256, 256, seg, 1, C.byref(hp), 256, None) == -4
    seg = (L.LoraSegment * 1)(L.LoraSegment(0, 8, 5))
    assert lib.lora_adamw_step(256, 256, 256, 256, seg, 1, C.byref(hp), 256, None) == -1
    assert lib.lora_adamw_step(256, 256, 256, 256, seg, 0, C.byref(hp), 256, None) == -1
    hp0 = L.LoraAdamwHparams(1e-4, 0.9, 0.999, 1e-8, 0.01, 1.0, 0)
    seg = (L.LoraSegment * 1)(L.LoraSegment(0, 8, 0))
    assert lib.lora_adamw_step(256, 256, 256, 256, seg, 1, C.byref(hp0), 256, None) == -1
    assert lib.lora_grad_prepare(256, 10, 0, 1.0, 256, None, None, 256, 1 << 16, None) == -1
    assert lib.lora_grad_prepare(256, 10, 4, -1.0, 256, None, None, 256, 1 << 16, None) == -1
    assert lib.lora_grad_prepare(256, 10, 4, 1.0, 256, None, None, 256, 16, None) == -5


def _nb_need(W, N, K, r, S):
    """Workspace of one expansion job as the library lays it out: the split
    parts, the P partials, the G partials and the row sums of squares, each
    rounded up to 256 bytes."""
    a = lambda x: (x + 255) // 256 * 256
    RP = -(-r // 32) * 32
    Kp = -(-K // 32) * 32
    ns = -(-Kp // 3072)
    klen = -(-(-(-Kp // ns)) // 32) * 32
    ns = -(-Kp // klen)
    C_ = S * RP
    return (a(S * 3 * RP * Kp * 2) + a(ns * N * C_ * 4) + a(ns * 3 * S * RP * C_ * 4) +
            a(ns * N * 8))


@no_device
def test_dora_norm_batch_workspace_and_validation():
    lib = L.lib()
    bf = lambda W, **kw: _lin(w_dtype=L.BF16, W=W, **kw)
    # Two slots over one W share a job; a third linear over another W is its own.
    lins = [bf(256, in_dim=2048, out_dim=300, rank=16), bf(256, in_dim=2048, out_dim=300, rank=16),
            bf(512, in_dim=2048, out_dim=300, rank=16)]
    arr = (L.LoraLinear * 3)(*lins)
    assert lib.lora_dora_row_norms_batch_workspace_bytes(3, arr) == \
        _nb_need(256, 300, 2048, 16, 2) + _nb_need(512, 300, 2048, 16, 1)
    # Nine W matrices: two launches that reuse the workspace; the largest counts.
    many = (L.LoraLinear * 9)(*[bf(256 * (i + 1), in_dim=512, out_dim=64 + i, rank=8)
                                for i in range(9)])
    chunk1 = sum(_nb_need(0, 64 + i, 512, 8, 1) for i in range(8))
    assert lib.lora_dora_row_norms_batch_workspace_bytes(9, many) == chunk1
    # Linears the expansion does not take need only what lora_dora_row_norms needs.
    f32 = (L.LoraLinear * 1)(_lin(in_dim=9728, out_dim=64, rank=16))
    assert lib.lora_dora_row_norms_batch_workspace_bytes(1, f32) == \
        lib.lora_dora_row_norms_workspace_bytes(C.byref(f32[0]))
    assert lib.lora_dora_row_norms_batch_workspace_bytes(0, arr) == 0
    outs = (C.c_void_p * 3)(256, 256, 256)
    need = lib.lora_dora_row_norms_batch_workspace_bytes(3, arr)
    assert lib.lora_dora_row_norms_batch(0, arr, outs, 256, need, None) == -1
    assert lib.lora_dora_row_norms_batch(3, arr, outs, 256, need - 1, None) == -5
    assert lib.lora_dora_row_norms_batch(3, arr, outs, None, need, None) == -5
    assert lib.lora_dora_row_norms_batch(3, arr, outs, 264, need, None) == -4
    bad = (L.LoraLinear * 3)(lins[0], lins[1], bf(512, in_dim=2048, out_dim=300, rank=200))
    assert lib.lora_dora_row_norms_batch(3, bad, outs, 256, need, None) == -2
    assert lib.lora_dora_row_norms_batch(3, arr, (C.c_void_p * 3)(256, None, 256), 256, need,
                                         None) == -1


def test_binding_checks_factor_shapes_against_w():
    """make_linear refuses factors that disagree with W's shape, on the host:
    the kernels size every access from the descriptor alone."""
    W = torch.zeros(64, 32)
    with pytest.raises(ValueError, match="B must be"):
        L.make_linear(W, torch.zeros(4, 32), torch.zeros(16, 4), 1.0, 8)
    with pytest.raises(ValueError, match="A must be"):
        L.make_linear(W, torch.zeros(4, 16), torch.zeros(64, 4), 1.0, 8)
    with pytest.raises(ValueError, match="dora_mag"):
        L.make_linear(W, torch.zeros(4, 32), torch.zeros(64, 4), 1.0, 8, torch.zeros(63))


@pytest.mark.parametrize("fmt", sorted(L.Q_FORMATS))
@pytest.mark.parametrize("N,K", [(8, 256), (264, 512), (4096, 2560)])
def test_qweight_layout_holds_the_documented_planes(fmt, N, K):
    """Plane offsets are 256-byte aligned, in table order, each plane fits
    before the next one, and the total covers the last."""
    from oracle import quant as Q
    if K % Q.SUPER[fmt]:
        assert L.lib().lora_qweight_layout(L.Q_FORMATS[fmt][0], N, K, None) == 0
        return
    total, offs = L.lora_qweight_layout(fmt, N, K)
    shapes = Q.plane_shapes(fmt, N, K)
    names = L.Q_FORMATS[fmt][1]
    assert list(names) == list(shapes)
    ends = offs[1:] + [total]
    for name, off, end in zip(names, offs, ends):
        dt, shp = shapes[name]
        nbytes = int(np.prod(shp)) * np.dtype(dt).itemsize
        assert off % 256 == 0 and off + nbytes <= end and end - (off + nbytes) < 256
    assert total % 256 == 0


def test_qweight_layout_rejects_non_block_shapes():
    code = L.Q_FORMATS["q6_k"][0]
    assert L.lib().lora_qweight_layout(code, 16, 128, None) == 0
    assert L.lib().lora_qweight_layout(code, 0, 256, None) == 0
    assert L.lib().lora_qweight_layout(L.BF16, 16, 256, None) == 0


def test_bf16_config_control_rejects_unknown_configurations():
    lib = L.lib()
    assert lib.lora_set_bf16_config(6) == -1
    assert lib.lora_set_bf16_config(-2) == -1
    assert lib.lora_set_bf16_config(-1) == 0
