"""Workload definitions and seeded synthetic inputs.

This module holds data only: shapes, hyper-parameters and seeded random
tensors.  It contains none of the method's arithmetic, so that both the HIP
path and the CPU oracle (used by the tests) can take their inputs from it.

Every tensor is drawn from ``torch.Generator`` seeded by a SeedSequence over
``(workload, slot, layer, projection, chunk, kind)``.  A tensor is a pure
function of that key and of the device it is drawn on (torch's CPU and GPU
generators produce different streams), so tests draw small cases on the CPU
and upload them, and large cases on the GPU and copy the sampled slices back.

Distributions (the workloads' own where given; otherwise the same as the
other workloads): W ~ N(0, 0.02); X ~ N(0, 1); dY ~ N(0, 1) or N(0, 0.01);
A ~ U(-1/sqrt(K), 1/sqrt(K)) (Kaiming-uniform for fan-in K); B ~ N(0, 0.01),
nonzero so that the A gradient is exercised.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = [
    "Projection",
    "LoraConfig",
    "CONFIGS",
    "get_config",
    "tensor_seed",
    "draw",
    "linear_inputs",
    "qweight_planes",
]


@dataclass(frozen=True)
class Projection:
    """A frozen projection: name, canonical ordinal (wq..wdown = 0..6), K -> N."""
    name: str
    ordinal: int
    in_dim: int
    out_dim: int
    x_group: int  # projections with equal x_group in a layer read the same X


@dataclass(frozen=True)
class LoraConfig:
    number: int
    name: str
    layers: int
    projections: tuple
    tokens: int                 # T, tokens per chunk
    chunks: int = 1             # G, accumulation chunks per update
    slots: int = 1              # S, independent adapter slots
    rank: int = 8
    alpha: float = 16.0
    scaling: str = "standard"   # or "rslora"
    w_dtype: str = "f32"        # "bf16", or a block-quantized format (bench --w-format)
    w_std: float = 0.02
    x_std: float = 1.0
    dy_std: float = 1.0
    b_std: float = 0.01
    dropout: float = 0.0
    seeds: tuple = (1234,)      # dropout seed per slot
    lr: float = 1e-4
    weight_decay: float = 0.01
    max_norm: float = 1.0
    plus_ratio: float = 1.0
    schedule: str = "constant"  # or "cosine"
    warmup: int = 0
    total_updates: int = 100
    lr_min: float = 0.0
    dora: bool = False
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8

    @property
    def tokens_per_step(self) -> int:
        return self.tokens * self.chunks * self.slots

    def shrink(self, **kw) -> "LoraConfig":
        return replace(self, **kw)


_TINYLLAMA = (
    Projection("wq", 0, 2048, 2048, 0),
    Projection("wv", 2, 2048, 256, 0),
)

_QWEN3_4B = (
    Projection("wq", 0, 2560, 4096, 0),
    Projection("wk", 1, 2560, 1024, 0),
    Projection("wv", 2, 2560, 1024, 0),
    Projection("wo", 3, 4096, 2560, 1),
    Projection("wgate", 4, 2560, 9728, 2),
    Projection("wup", 5, 2560, 9728, 2),
    Projection("wdown", 6, 9728, 2560, 3),
)

CONFIGS = {
    1: LoraConfig(1, "single-64x64-f32-r4", layers=1,
                  projections=(Projection("w", 0, 64, 64, 0),),
                  tokens=32, rank=4, alpha=8.0, dy_std=1.0,
                  lr=1e-4, weight_decay=0.01, max_norm=1.0),
    2: LoraConfig(2, "tinyllama-wq-wv-f32-r8", layers=22, projections=_TINYLLAMA,
                  tokens=128, chunks=4, rank=8, alpha=16.0, dy_std=1e-2,
                  dropout=0.05, seeds=(1234,), max_norm=1.0),
    3: LoraConfig(3, "wide-4096-f32-r16", layers=1,
                  projections=(Projection("w", 0, 4096, 4096, 0),),
                  tokens=1536, rank=16, alpha=32.0, dy_std=1.0,
                  plus_ratio=16.0, weight_decay=0.1),
    4: LoraConfig(4, "qwen3-4b-all-linear-bf16-r32-rslora", layers=36,
                  projections=_QWEN3_4B, tokens=4096, rank=32, alpha=32.0,
                  scaling="rslora", w_dtype="bf16", dy_std=1e-2,
                  schedule="cosine", warmup=10, total_updates=100),
    5: LoraConfig(5, "qwen3-4b-dora-bf16-r64-2slot", layers=36,
                  projections=_QWEN3_4B, tokens=2048, chunks=2, slots=2,
                  rank=64, alpha=64.0, w_dtype="bf16", dy_std=1e-2,
                  dropout=0.1, seeds=(1234, 1235), dora=True),
}


def get_config(n: int) -> LoraConfig:
    return CONFIGS[int(n)]


_KIND = {"W": 0, "X": 1, "dY": 2, "A": 3, "B": 4}


def tensor_seed(cfg: int, slot: int, layer: int, proj: int, chunk: int, kind: str) -> int:
    """63-bit seed for one tensor, from numpy's SeedSequence over the key."""
    ss = np.random.SeedSequence([cfg, slot, layer, proj, chunk, _KIND[kind]])
    return int(ss.generate_state(1, np.uint64)[0] >> np.uint64(1))


def draw(shape, key: tuple, dist: str, param: float, device="cpu") -> torch.Tensor:
    """Seeded float32 tensor: dist 'normal' (std=param) or 'uniform' (+-param)."""
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(*key))
    if dist == "normal":
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return t.mul_(param)
    if dist == "uniform":
        t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        return t.mul_(2.0 * param).sub_(param)
    raise ValueError(dist)


def _gen(key: tuple, plane: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(*key, 1 + plane, "W"))
    return g


def _ints(shape, lo, hi, dtype, key, plane, device):
    """Seeded integers, uniform in [lo, hi)."""
    t = torch.randint(lo, hi, shape, generator=_gen(key, plane, device), device=device,
                      dtype=torch.int32)
    return t.to(dtype)


def _halves(shape, lo, hi, key, plane, device):
    """Seeded float16 values, uniform in [lo, hi)."""
    t = torch.rand(shape, generator=_gen(key, plane, device), device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo).to(torch.float16)


def qweight_planes(fmt: str, N: int, K: int, key: tuple, device="cpu") -> dict:
    """Seeded planes of a block-quantized W [N, K] (formats and plane layouts
    as in include/lora.h), drawn directly: codes uniform over their range,
    fp16 scales uniform in a band chosen so that the decoded weights spread
    about as widely as W ~ N(0, 0.02).  key = (workload, slot, layer, proj);
    field i is drawn from the "W" kind with chunk index 1 + i."""
    if fmt == "q8_0":
        return {"qs": _ints((N, K), -127, 128, torch.int8, key, 0, device),
                "d": _halves((N, K // 32), 2.0e-4, 3.4e-4, key, 1, device)}
    if fmt == "q4_0":
        return {"qs": _ints((N, K // 2), 0, 256, torch.uint8, key, 0, device),
                "d": _halves((N, K // 32), 3.2e-3, 5.4e-3, key, 1, device)}
    if fmt == "q4_k":
        sc = _ints((N, K // 32, 1), 32, 64, torch.uint8, key, 1, device)
        mn = _ints((N, K // 32, 1), 0, 64, torch.uint8, key, 2, device)
        d = _halves((N, K // 256, 1), 6.8e-5, 1.1e-4, key, 3, device)
        dmin = _halves((N, K // 256, 1), 7.5e-4, 1.25e-3, key, 4, device)
        return {"qs": _ints((N, K // 2), 0, 256, torch.uint8, key, 0, device),
                "sm": torch.cat([sc, mn], dim=2), "dm": torch.cat([d, dmin], dim=2)}
    if fmt == "q6_k":
        return {"ql": _ints((N, K // 2), 0, 256, torch.uint8, key, 0, device),
                "qh": _ints((N, K // 4), 0, 256, torch.uint8, key, 1, device),
                "sc": _ints((N, K // 16), -32, 32, torch.int8, key, 2, device),
                "d": _halves((N, K // 256), 2.0 ** -14, 2.0 ** -13, key, 3, device)}
    raise ValueError(f"unknown format {fmt!r}")


def linear_inputs(cfg: LoraConfig, layer: int, proj: Projection, slot: int = 0,
                  chunks=None, device="cpu", tokens=None) -> dict:
    """All seeded inputs of one linear: W, A, B and per-chunk X, dY.

    W is returned as float32 and, for bf16 workloads, also as ``W_bf16`` (the
    float32 tensor holds exactly the bf16 values).  X is keyed by the
    projection's x_group so that projections sharing an input read equal X.
    """
    T = cfg.tokens if tokens is None else tokens
    K, N, r = proj.in_dim, proj.out_dim, cfg.rank
    n = cfg.number
    out = {}
    W = draw((N, K), (n, 0, layer, proj.ordinal, 0, "W"), "normal", cfg.w_std, device)
    if cfg.w_dtype == "bf16":
        Wb = W.to(torch.bfloat16)
        out["W_bf16"] = Wb
        W = Wb.to(torch.float32)
    out["W"] = W
    out["A"] = draw((r, K), (n, slot, layer, proj.ordinal, 0, "A"), "uniform",
                    1.0 / math.sqrt(K), device)
    out["B"] = draw((N, r), (n, slot, layer, proj.ordinal, 0, "B"), "normal",
                    cfg.b_std, device)
    xs, dys = [], []
    for c in range(cfg.chunks if chunks is None else chunks):
        xs.append(draw((T, K), (n, slot, layer, 100 + proj.x_group, c, "X"),
                       "normal", cfg.x_std, device))
        dys.append(draw((T, N), (n, slot, layer, proj.ordinal, c, "dY"),
                        "normal", cfg.dy_std, device))
    out["X"] = xs
    out["dY"] = dys
    return out
