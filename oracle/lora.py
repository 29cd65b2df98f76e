"""Plain float64 CPU oracle for the LoRA-linear forward, backward and step.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg; never by the product path.

Sources (page title, then section):

* "8. LoRA Fundamentals: The Math and the Architecture Support Matrix"
  (Juno docs), section "How it works": the adapted weight ``W + scale*B*A``
  with A ``rank x inDim`` and B ``outDim x rank``; ``scale = alpha/rank`` or
  ``alpha/sqrt(rank)`` (rsLoRA); B starts at zero; canonical DoRA rescales each
  output row by ``magnitude / ||W + Delta||`` with the norm detached.
  Section "The training loop": sum over chunks, divide by prediction tokens,
  clip by global L2 norm, one AdamW step per group; decay on A only.
  Section "Training decisions": the frozen transpose product ``W^T g``;
  accumulation equals training on the concatenated chunk.
* "4.3. Training Guide" (Juno docs), sections "Gradient accumulation",
  "Optimizer", "Schedules", "Dropout", "Gradient clipping".
* "Backward Bug Hunts and Vulkan Tiled GEMM: Pi-Train LoRA SFT Hardening",
  section "Bug #1": the LoRA-A gradient factor ``B^T @ grad``, zero while B is
  zero.
* "Multi-LoRA Training Example (fully-async)", section "Design (decoupled
  per-adapter optimizers)": each slot has its own Adam state, step count and
  clipping.

Readings taken where the pages leave a step open (each is listed in the
design notes of the repository with its reason):

* Row-major layout: X ``[T,K]``, W ``[N,K]``, A ``[r,K]``, B ``[N,r]``,
  U = X~ A^T ``[T,r]``, V = g B ``[T,r]``, Y, dY, Z ``[T,N]``.
* Dropout is element-wise over ``[T,K]`` on the LoRA-branch input only; the
  hash chains SplitMix64's output function over (seed, step, accumulation
  ordinal, layer, projection, token, feature) and keeps an element when the
  top 24 bits are ``>= round(p * 2**24)``; the kept value is scaled by
  ``float32(1/(1-p))``.
* The clip compares ``max_norm`` with ``||g|| / Npred`` and clips only when it
  is strictly greater; the combined scale is rounded once to float32.
* AdamW: beta1 0.9, beta2 0.999, eps 1e-8 outside the square root, bias
  corrected moments; decay ``lr * wd * A_old`` on A only; B's rate is
  ``lr * ratio``; the DoRA magnitude is trained at the base rate, undecayed.
* Warmup-cosine: linear warmup ``lr*(k+1)/Wu`` then cosine from lr to lr_min
  over ``total - Wu`` updates, k being the 0-based update index.
* DoRA: magnitude trainable; row norm refreshed at init and after each update.

Pinning (tests under ``tests/test_oracle_*.py`` pin each function to something
other than itself):

* ``mix64`` -- published SplitMix64 reference outputs (golden file).
* ``dropout_keep`` -- keep-fraction statistics, per-key sensitivity, rerun
  equality, p = 0 reduces to all-keep.  The chaining order itself is a
  declared reading: no source fixes those bits ("parity unpinned" for the
  exact bit pattern beyond the mixer and the statistics).
* ``forward``/``backward`` -- B = 0 exact no-op, merged-weight forward, central
  finite differences, float64 ``torch.autograd``, adjointness, DoRA closed form.
* ``grad_prepare`` -- clipped norm equals max_norm, unclipped closed form,
  non-finite veto.
* ``adamw_update`` -- first-step closed form and ``torch.optim.AdamW``.
* ``lr_at`` -- schedule closed forms (warmup end, midpoint, end).
* ``dora_row_norms`` -- ``numpy.linalg.norm`` of the merged weight; B = 0
  gives the plain row norms.
* ``bf16_round`` -- hand-worked round-to-nearest-even cases (ties both ways,
  carry into the exponent).
* ``merge`` -- B = 0 returns W itself (RMSE 0 for bf16 W); ``X merged^T``
  equals ``forward``'s Y (plain and DoRA); the RMSE of a matrix of ties
  has a closed form.
* ``train_step`` -- accumulation over G chunks equals one concatenated chunk;
  seeded reruns give identical adapters.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "scaling",
    "splitmix64_next",
    "mix64",
    "dropout_threshold",
    "dropout_scale",
    "dropout_keep",
    "forward",
    "backward",
    "grad_prepare",
    "adamw_update",
    "lr_at",
    "dora_row_norms",
    "bf16_round",
    "merge",
    "SlotState",
    "train_step",
]

F64 = np.float64
_U64 = np.uint64
_MASK64 = (1 << 64) - 1

# SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014): state increment and output-function constants.
_SM_GAMMA = 0x9E3779B97F4A7C15
_SM_M1 = 0xBF58476D1CE4E5B9
_SM_M2 = 0x94D049BB133111EB


# --------------------------------------------------------------------------
# scaling -- "8. LoRA Fundamentals", "How it works"
# --------------------------------------------------------------------------
def scaling(alpha: float, rank: int, mode: str = "standard") -> float:
    """LoRA scale: alpha/rank (standard) or alpha/sqrt(rank) (rsLoRA)."""
    if rank <= 0:
        raise ValueError("rank must be positive")
    if mode == "standard":
        return float(alpha) / float(rank)
    if mode == "rslora":
        return float(alpha) / math.sqrt(float(rank))
    raise ValueError(f"unknown scaling mode {mode!r}")


# --------------------------------------------------------------------------
# dropout hash -- "4.3. Training Guide", "Dropout"
# --------------------------------------------------------------------------
def splitmix64_next(state: int) -> tuple[int, int]:
    """One SplitMix64 step on a Python int: returns (next_state, output)."""
    state = (state + _SM_GAMMA) & _MASK64
    z = state
    z = ((z ^ (z >> 30)) * _SM_M1) & _MASK64
    z = ((z ^ (z >> 27)) * _SM_M2) & _MASK64
    return state, z ^ (z >> 31)


def mix64(x):
    """SplitMix64 output for state ``x`` (uint64 numpy array or scalar).

    Equal to ``splitmix64_next(x)[1]``; written on uint64 arrays, whose
    products wrap modulo 2**64.
    """
    z = np.asarray(x, dtype=_U64) + _U64(_SM_GAMMA)
    z = (z ^ (z >> _U64(30))) * _U64(_SM_M1)
    z = (z ^ (z >> _U64(27))) * _U64(_SM_M2)
    return z ^ (z >> _U64(31))


def dropout_threshold(p: float) -> int:
    """Integer keep threshold on 24 hash bits; p is taken as a float32."""
    p32 = float(np.float32(p))
    if not (0.0 <= p32 < 1.0):
        raise ValueError("dropout p must lie in [0, 1)")
    return int(round(p32 * float(1 << 24)))


def dropout_scale(p: float) -> float:
    """Inverted-dropout multiplier float32(1/(1-p)), returned as a float."""
    p32 = float(np.float32(p))
    return float(np.float32(1.0 / (1.0 - p32)))


def dropout_keep(seed: int, step: int, ordinal: int, layer: int, proj: int,
                 tokens: int, in_dim: int, p: float) -> np.ndarray:
    """Keep mask ``[tokens, in_dim]`` (bool) for one projection of one chunk.

    Stateless: a chain of SplitMix64 outputs over (seed, optimizer step,
    accumulation ordinal, layer, projection, token row, feature column).
    An element is kept when the top 24 bits reach ``round(p * 2**24)``.
    """
    thr = dropout_threshold(p)
    with np.errstate(over="ignore"):
        h = mix64(_U64(seed & _MASK64))
        for key in (step, ordinal, layer, proj):
            h = mix64(h ^ _U64(key & _MASK64))
        rows = mix64(h ^ np.arange(tokens, dtype=_U64))            # [T]
        bits = mix64(rows[:, None] ^ np.arange(in_dim, dtype=_U64)[None, :])
    top24 = (bits >> _U64(40)).astype(np.int64)
    return top24 >= thr


# --------------------------------------------------------------------------
# forward / backward -- "8. LoRA Fundamentals", "How it works";
# "Backward Bug Hunts ...", "Bug #1"
# --------------------------------------------------------------------------
def _masked(X, keep, keep_scale):
    X = np.asarray(X, dtype=F64)
    if keep is None:
        return X
    return np.where(keep, X * F64(keep_scale), F64(0.0))


def forward(X, W, A, B, s, keep=None, keep_scale=1.0, mag=None, norm=None):
    """Adapted linear over one chunk.

    ``U = X~ A^T``;  ``Z = X W^T + s U B^T``;  ``Y = Z`` or, for DoRA,
    ``Y = (mag / norm) * Z`` per output column.  X~ is X with the dropout
    mask and scale applied (the LoRA branch only).  Returns (Y, U, Z).
    """
    X = np.asarray(X, dtype=F64)
    W = np.asarray(W, dtype=F64)
    A = np.asarray(A, dtype=F64)
    B = np.asarray(B, dtype=F64)
    Xt = _masked(X, keep, keep_scale)
    U = Xt @ A.T
    Z = X @ W.T + F64(s) * (U @ B.T)
    if mag is None:
        return Z, U, Z
    c = np.asarray(mag, dtype=F64) / np.asarray(norm, dtype=F64)
    return Z * c[None, :], U, Z


def backward(X, dY, W, A, B, s, U, keep=None, keep_scale=1.0,
             mag=None, norm=None, Z=None):
    """Gradients of one chunk.

    With ``g = dY`` (DoRA: ``g = dY * mag/norm``, the norm being detached):
    ``V = g B``;  ``dX = g W + s (V A) * mask * scale``;
    ``dB = s g^T U``;  ``dA = s V^T X~``;  DoRA ``dm_n = sum_t dY Z / norm_n``.
    Returns dict with dX, dA, dB and (DoRA) dmag.
    """
    dY = np.asarray(dY, dtype=F64)
    W = np.asarray(W, dtype=F64)
    A = np.asarray(A, dtype=F64)
    B = np.asarray(B, dtype=F64)
    U = np.asarray(U, dtype=F64)
    out = {}
    if mag is not None:
        nrm = np.asarray(norm, dtype=F64)
        g = dY * (np.asarray(mag, dtype=F64) / nrm)[None, :]
        out["dmag"] = (dY * np.asarray(Z, dtype=F64)).sum(axis=0) / nrm
    else:
        g = dY
    V = g @ B
    lora = F64(s) * (V @ A)
    if keep is not None:
        lora = np.where(keep, lora * F64(keep_scale), F64(0.0))
    out["dX"] = g @ W + lora
    out["dB"] = F64(s) * (g.T @ U)
    out["dA"] = F64(s) * (V.T @ _masked(X, keep, keep_scale))
    out["V"] = V
    return out


# --------------------------------------------------------------------------
# gradient preparation -- "4.3. Training Guide", "Gradient clipping" and
# "Gradient accumulation"
# --------------------------------------------------------------------------
def grad_prepare(grads, n_pred: int, max_norm: float) -> dict:
    """Two passes over the slot's summed gradients.

    Pass 1: squared L2 norm accumulated in double and a finiteness check.
    Pass 2: ``norm = sqrt(ss) / Npred``; ``clip = max_norm / norm`` when
    ``max_norm > 0`` and ``norm > max_norm``, else 1; one combined scale
    ``c = float32(clip / Npred)``.  Non-finite input vetoes the update.
    """
    if n_pred <= 0:
        raise ValueError("n_pred must be positive")
    flat = [np.asarray(g, dtype=F64).ravel() for g in grads]
    finite = all(bool(np.isfinite(f).all()) for f in flat)
    if not finite:
        return {"finite": False, "norm": float("nan"), "clip": float("nan"),
                "scale": float("nan")}
    ss = 0.0
    for f in flat:
        ss += float(np.dot(f, f))
    norm = math.sqrt(ss) / float(n_pred)
    mn = float(np.float32(max_norm))
    clip = mn / norm if (mn > 0.0 and norm > mn) else 1.0
    scale = float(np.float32(clip / float(n_pred)))
    return {"finite": True, "norm": norm, "clip": clip, "scale": scale}


# --------------------------------------------------------------------------
# AdamW -- "4.3. Training Guide", "Optimizer"; "8. LoRA Fundamentals",
# "The training loop" and "Training decisions"
# --------------------------------------------------------------------------
def adamw_update(theta, g, m, v, kind: str, lr: float, t: int, scale: float,
                 beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                 plus_ratio=1.0):
    """One decoupled AdamW update of one tensor; returns (theta, m, v).

    The moments see the prepared gradient ``g' = g * scale`` (no decay term).
    A is decayed by ``lr * wd * theta_old`` (uncorrected rate, pre-update
    value); B moves at ``lr * plus_ratio`` and is never decayed; the DoRA
    magnitude ("mag") moves at ``lr`` and is never decayed.
    """
    if kind not in ("A", "B", "mag"):
        raise ValueError(kind)
    theta = np.asarray(theta, dtype=F64)
    gp = np.asarray(g, dtype=F64) * F64(scale)
    m = F64(beta1) * np.asarray(m, dtype=F64) + F64(1.0 - beta1) * gp
    v = F64(beta2) * np.asarray(v, dtype=F64) + F64(1.0 - beta2) * gp * gp
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    rate = lr * plus_ratio if kind == "B" else lr
    new = theta - F64(rate) * m_hat / (np.sqrt(v_hat) + F64(eps))
    if kind == "A":
        new = new - F64(lr * weight_decay) * theta
    return new, m, v


# --------------------------------------------------------------------------
# schedule -- "4.3. Training Guide", "Schedules"
# --------------------------------------------------------------------------
def lr_at(k: int, lr: float, schedule: str = "constant", warmup: int = 0,
          total: int = 100, lr_min: float = 0.0) -> float:
    """Learning rate for the 0-based optimizer-update index ``k``."""
    if schedule == "constant":
        return float(lr)
    if schedule != "cosine":
        raise ValueError(schedule)
    if k < warmup:
        return float(lr) * (k + 1) / warmup
    progress = min(1.0, (k - warmup) / max(1, total - warmup))
    return lr_min + 0.5 * (lr - lr_min) * (1.0 + math.cos(math.pi * progress))


# --------------------------------------------------------------------------
# DoRA row norms -- "8. LoRA Fundamentals", "How it works"
# --------------------------------------------------------------------------
def dora_row_norms(W, A=None, B=None, s=1.0):
    """``||W_i + s (B A)_i||_2`` for every output row i (``||W_i||`` if A is None)."""
    W = np.asarray(W, dtype=F64)
    if A is None:
        M = W
    else:
        M = W + F64(s) * (np.asarray(B, dtype=F64) @ np.asarray(A, dtype=F64))
    return np.sqrt((M * M).sum(axis=1))


# --------------------------------------------------------------------------
# Merge for export -- "8. LoRA Fundamentals", "How it works" (the effective
# weight W + scale*B*A, merged in F32; DoRA's per-row rescale) and "Profiling
# with --jfr" (the merge reports the RMSE of requantising the merged weight)
# --------------------------------------------------------------------------
def bf16_round(x):
    """Round float32 values to bfloat16, to nearest with ties to even,
    returned as float64.  (NaN and infinities are not handled.)"""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return r.astype(np.uint32).view(np.float32).astype(F64)


def merge(W, A, B, s, mag=None, norm=None, out="f32"):
    """Merged weight ``c_i (W + s B A)_i`` (``c = mag/norm`` for DoRA, else 1),
    stored as float32 (``out="f32"``) or rounded to bfloat16 from its float32
    value (``out="bf16"``).  Returns ``(W_out, rmse)`` where ``rmse`` is the
    root mean square of ``W_out`` minus the float32 merged weight over all
    elements (0 for float32 output)."""
    M = np.asarray(W, dtype=F64) + F64(s) * (np.asarray(B, dtype=F64) @ np.asarray(A, dtype=F64))
    if mag is not None:
        M = M * (np.asarray(mag, dtype=F64) / np.asarray(norm, dtype=F64))[:, None]
    m32 = M.astype(np.float32).astype(F64)
    if out == "f32":
        return m32, 0.0
    if out != "bf16":
        raise ValueError(out)
    q = bf16_round(m32)
    return q, float(np.sqrt(np.mean((q - m32) ** 2)))


# --------------------------------------------------------------------------
# whole optimizer step for one adapter slot
# --------------------------------------------------------------------------
@dataclass
class SlotState:
    """Trainable state of one adapter slot.

    ``params[key]`` holds {"A", "B"} (and "mag" for DoRA) per linear key
    ``(layer, proj)``; ``m``/``v`` mirror it; ``t`` counts applied updates;
    ``k`` is the 0-based index of the next update (schedule and dropout step).
    """
    params: dict
    m: dict = field(default_factory=dict)
    v: dict = field(default_factory=dict)
    norms: dict = field(default_factory=dict)
    t: int = 0
    k: int = 0


def train_step(state: SlotState, linears: dict, chunks: list, hp: dict,
               keep_outputs: bool = False) -> dict:
    """One optimizer update of a slot over G chunks.

    ``linears[key]`` = frozen W ``[N,K]`` for key ``(layer, proj)``.
    ``chunks[g][key]`` = (X, dY) for chunk g.  ``hp`` holds: s, p, seed,
    n_pred, max_norm, lr (already scheduled for update ``state.k``), beta1,
    beta2, eps, weight_decay, plus_ratio, dora (bool).

    Order: every chunk runs forward over all linears then backward, gradients
    are summed over chunks; then prepare, AdamW, and (DoRA) the row-norm
    refresh.  A non-finite gradient leaves the state untouched.
    """
    keys = sorted(linears)
    dora = bool(hp.get("dora", False))
    p = float(hp.get("p", 0.0))
    ks = dropout_scale(p) if p > 0 else 1.0
    grads = {key: {} for key in keys}
    outputs = []
    for ordinal, chunk in enumerate(chunks):
        saved = {}
        outs = {}
        for key in keys:
            X, _ = chunk[key]
            W = linears[key]
            pr = state.params[key]
            keep = None
            if p > 0:
                keep = dropout_keep(hp["seed"], state.k, ordinal, key[0], key[1],
                                    X.shape[0], X.shape[1], p)
            mag = pr["mag"] if dora else None
            nrm = state.norms[key] if dora else None
            Y, U, Z = forward(X, W, pr["A"], pr["B"], hp["s"], keep, ks, mag, nrm)
            saved[key] = (U, Z, keep)
            outs[key] = {"Y": Y, "U": U}
        for key in reversed(keys):
            X, dY = chunk[key]
            U, Z, keep = saved[key]
            pr = state.params[key]
            mag = pr["mag"] if dora else None
            nrm = state.norms[key] if dora else None
            gr = backward(X, dY, linears[key], pr["A"], pr["B"], hp["s"], U,
                          keep, ks, mag, nrm, Z)
            outs[key]["dX"] = gr["dX"]
            for name, gname in (("A", "dA"), ("B", "dB"), ("mag", "dmag")):
                if gname in gr:
                    acc = grads[key].get(name)
                    grads[key][name] = gr[gname] if acc is None else acc + gr[gname]
        if keep_outputs:
            outputs.append(outs)
    flat = [grads[key][name] for key in keys for name in sorted(grads[key])]
    prep = grad_prepare(flat, hp["n_pred"], hp["max_norm"])
    result = {"prep": prep, "grads": grads, "outputs": outputs, "vetoed": False}
    if not prep["finite"]:
        result["vetoed"] = True
        return result
    t = state.t + 1
    for key in keys:
        for name, g in grads[key].items():
            th = state.params[key][name]
            m0 = state.m.get(key, {}).get(name, np.zeros_like(th, dtype=F64))
            v0 = state.v.get(key, {}).get(name, np.zeros_like(th, dtype=F64))
            new, m1, v1 = adamw_update(
                th, g, m0, v0, name, hp["lr"], t, prep["scale"],
                hp.get("beta1", 0.9), hp.get("beta2", 0.999), hp.get("eps", 1e-8),
                hp.get("weight_decay", 0.0), hp.get("plus_ratio", 1.0))
            state.params[key][name] = new
            state.m.setdefault(key, {})[name] = m1
            state.v.setdefault(key, {})[name] = v1
    if dora:
        for key in keys:
            pr = state.params[key]
            state.norms[key] = dora_row_norms(linears[key], pr["A"], pr["B"], hp["s"])
    state.t = t
    state.k += 1
    return result
