"""Block-quantized frozen weights: plain float64 dequantisation.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg; never by the product path.

Sources (page title, then section):

* "8. LoRA Fundamentals: The Math and the Architecture Support Matrix"
  (Juno docs), opening paragraph: adapters are trained over a quantized GGUF
  base model.  Section "Training decisions" ("Frozen weights in backward"):
  the transpose product ``W^T g`` reads the same frozen weights, dequantised.
* "Backward Bug Hunts and Vulkan Tiled GEMM: Pi-Train LoRA SFT Hardening",
  section "The fix": the Q4_0, Q4_K and Q6_K frozen-weight backward paths,
  which dominate the step time.

The pages name the formats but not their block layouts.  The arithmetic
below is the published definition of each format (the GGUF block types of
the same names); the storage is our own, one array per field ("planes")
instead of interleaved block records.  Every row of W ``[N, K]`` is cut into
consecutive blocks along K, and every element decodes to ``a * q + b`` with
``a``, ``b`` fixed per (row, sub-block):

============  =========  ===========================================  ==============================
format        block      planes (numpy dtype, shape)                  value
============  =========  ===========================================  ==============================
``q8_0``      32         qs int8 [N,K]; d float16 [N,K/32]            ``d * q``
``q4_0``      32         qs uint8 [N,K/2]; d float16 [N,K/32]         ``d * (q - 8)``
``q4_k``      256 = 8x32 qs uint8 [N,K/2]; sm uint8 [N,K/32,2]        ``d*sc * q - dmin*mn``
                         (sc, mn < 64); dm float16 [N,K/256,2] (d, dmin)
``q6_k``      256 = 16x16 ql uint8 [N,K/2]; qh uint8 [N,K/4];          ``d*sc * (q - 32)``,
                         sc int8 [N,K/16]; d float16 [N,K/256]        ``q = ql | qh << 4``
============  =========  ===========================================  ==============================

Packed codes: element ``2j`` of a row is the low nibble of byte ``j`` of its
4-bit plane and element ``2j+1`` the high nibble; in ``qh`` element ``4j+i``
holds bits ``2i..2i+1`` of byte ``j``.

Pinning (``tests/test_oracle_pins.py``): codes laid out by an independent
packer from a closed-form code pattern decode to the closed-form values;
neutral codes give exactly zero; q4_0 equals q4_k with unit sub-scales and
``dmin = 8 d``; q6_k equals q8_0 with codes shifted by 32 and ``d8 = d*sc``;
sub-block scales reach exactly their own 32 (or 16) elements.
"""

from __future__ import annotations

import numpy as np

FORMATS = ("q8_0", "q4_0", "q4_k", "q6_k")

# elements per block carrying the fp16 scale(s); elements per sub-block
SUPER = {"q8_0": 32, "q4_0": 32, "q4_k": 256, "q6_k": 256}
SUB = {"q8_0": 32, "q4_0": 32, "q4_k": 32, "q6_k": 16}


def _nibbles(qs):
    """uint8 [N, K/2] -> codes [N, K]: low nibble first."""
    qs = np.asarray(qs, dtype=np.uint8)
    out = np.empty((qs.shape[0], 2 * qs.shape[1]), dtype=np.int64)
    out[:, 0::2] = qs & 0x0F
    out[:, 1::2] = qs >> 4
    return out


def _crumbs(qh):
    """uint8 [N, K/4] -> 2-bit fields [N, K]: bits 0-1 first."""
    qh = np.asarray(qh, dtype=np.uint8).astype(np.int64)
    out = np.empty((qh.shape[0], 4 * qh.shape[1]), dtype=np.int64)
    for i in range(4):
        out[:, i::4] = (qh >> (2 * i)) & 0x3
    return out


def _per_element(x, size):
    """[N, K/size] -> [N, K], each value repeated over its `size` elements."""
    return np.repeat(np.asarray(x, dtype=np.float64), size, axis=1)


def dequantize(fmt: str, planes: dict) -> np.ndarray:
    """float64 W [N, K] of a block-quantized weight (the table above)."""
    if fmt == "q8_0":
        q = np.asarray(planes["qs"], dtype=np.int8).astype(np.float64)
        return _per_element(planes["d"], 32) * q
    if fmt == "q4_0":
        q = _nibbles(planes["qs"]).astype(np.float64)
        return _per_element(planes["d"], 32) * (q - 8.0)
    if fmt == "q4_k":
        q = _nibbles(planes["qs"]).astype(np.float64)
        sm = np.asarray(planes["sm"], dtype=np.uint8)
        dm = np.asarray(planes["dm"], dtype=np.float16)
        d = _per_element(dm[:, :, 0], 256)
        dmin = _per_element(dm[:, :, 1], 256)
        sc = _per_element(sm[:, :, 0], 32)
        mn = _per_element(sm[:, :, 1], 32)
        return d * sc * q - dmin * mn
    if fmt == "q6_k":
        q = (_nibbles(planes["ql"]) | (_crumbs(planes["qh"]) << 4)).astype(np.float64)
        d = _per_element(planes["d"], 256)
        sc = _per_element(np.asarray(planes["sc"], dtype=np.int8), 16)
        return d * sc * (q - 32.0)
    raise ValueError(f"unknown format {fmt!r}")


def plane_shapes(fmt: str, N: int, K: int) -> dict:
    """Name -> (numpy dtype, shape) of each plane of an [N, K] weight."""
    if K % SUPER[fmt]:
        raise ValueError(f"{fmt} needs K divisible by {SUPER[fmt]}")
    if fmt == "q8_0":
        return {"qs": (np.int8, (N, K)), "d": (np.float16, (N, K // 32))}
    if fmt == "q4_0":
        return {"qs": (np.uint8, (N, K // 2)), "d": (np.float16, (N, K // 32))}
    if fmt == "q4_k":
        return {"qs": (np.uint8, (N, K // 2)), "sm": (np.uint8, (N, K // 32, 2)),
                "dm": (np.float16, (N, K // 256, 2))}
    if fmt == "q6_k":
        return {"ql": (np.uint8, (N, K // 2)), "qh": (np.uint8, (N, K // 4)),
                "sc": (np.int8, (N, K // 16)), "d": (np.float16, (N, K // 256))}
    raise ValueError(f"unknown format {fmt!r}")
