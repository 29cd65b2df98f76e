"""GPU parity: every C-ABI entry point against the float64 CPU oracle on the
same seeded inputs.

Bars: dropout masks bit-exact; float32-W paths max|gpu-ref|/max|ref| <= 1e-4;
bf16-W paths <= 2e-2 (the frozen products round X and dY to bf16 for MFMA).
"""

import hashlib
import math
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from oracle import quant as Q
from bwd_adamw_amd import lora as L
from bwd_adamw_amd import step as S
from bwd_adamw_amd import workloads as WL
from tests.helpers import np64, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL.update({f: TOL["bf16"] for f in Q.FORMATS})   # bf16 products on the decoded weights


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------- inputs ----
def _linear_case(T, K, N, r, w_dtype="f32", seed=0, x_std=1.0, dy_std=1.0, b_std=0.01,
                 device="cpu"):
    key = lambda kind, c=0: (900 + seed, 0, 0, 0, c, kind)
    W = WL.draw((N, K), key("W"), "normal", 0.02, device)
    out = {}
    if w_dtype in Q.FORMATS:
        planes = WL.qweight_planes(w_dtype, N, K, (900 + seed, 0, 0, 0))
        out["Wq"] = ("qweight", w_dtype, N, K, planes)
        W = torch.from_numpy(Q.dequantize(w_dtype, {k: v.numpy() for k, v in planes.items()}))
    elif w_dtype == "bf16":
        out["Wq"] = W.to(torch.bfloat16)
        W = out["Wq"].float()
    else:
        out["Wq"] = W
    out["W"] = W
    out["A"] = WL.draw((r, K), key("A"), "uniform", 1 / math.sqrt(K), device)
    out["B"] = WL.draw((N, r), key("B"), "normal", b_std, device)
    out["X"] = WL.draw((T, K), key("X"), "normal", x_std, device)
    out["dY"] = WL.draw((T, N), key("dY"), "normal", dy_std, device)
    return out


def _gpu(d):
    """Device copies; a quantized W is packed into the library's layout."""
    out = {}
    for k, v in d.items():
        if isinstance(v, tuple) and v[0] == "qweight":
            _, fmt, N, K, planes = v
            out[k] = L.qweight_pack(fmt, N, K, {n: t.to(DEV) for n, t in planes.items()})
        else:
            out[k] = v.to(DEV)
    return out


def _run_gpu(c, s, p=0.0, dkeys=(1234, 0, 0, 0, 0), dora=False, accumulate=False):
    g = _gpu(c)
    T, K = g["X"].shape
    N = g["W"].shape[0]
    r = g["A"].shape[0]
    mag = nrm = None
    if dora:
        mag = torch.empty(N, device=DEV)
        nrm = torch.empty(N, device=DEV)
        bare = L.make_linear(g["Wq"], None, None, s, T)
        L.lora_dora_row_norms(bare, mag)
        L.lora_dora_row_norms(L.make_linear(g["Wq"], g["A"], g["B"], s, T), nrm)
    lin = L.make_linear(g["Wq"], g["A"], g["B"], s, T, mag, nrm)
    ws = torch.empty(L.lora_workspace_bytes(lin), device=DEV, dtype=torch.uint8)
    drop = L.make_dropout(*dkeys, p) if p > 0 else None
    nanf = float("nan")
    Y = torch.full((T, N), nanf, device=DEV)
    U = torch.full((T, r), nanf, device=DEV)
    Z = torch.full((T, N), nanf, device=DEV) if dora else None
    L.lora_forward(lin, g["X"], Y, U, Z, drop, ws)
    dX = torch.full((T, K), nanf, device=DEV)
    dA = torch.full((r, K), nanf, device=DEV)
    dB = torch.full((N, r), nanf, device=DEV)
    dm = torch.full((N,), nanf, device=DEV) if dora else None
    L.lora_backward(lin, g["X"], g["dY"], U, Z, dX, dA, dB, dm, False, drop, ws)
    torch.cuda.synchronize()
    return dict(Y=Y, U=U, Z=Z, dX=dX, dA=dA, dB=dB, dmag=dm, mag=mag, norm=nrm, lin=lin, ws=ws, g=g)


def _oracle(c, s, p=0.0, dkeys=(1234, 0, 0, 0, 0), mag=None, nrm=None):
    X, W, A, B, dY = (np64(c[k]) for k in ("X", "W", "A", "B", "dY"))
    T, K = X.shape
    keep, ks = None, 1.0
    if p > 0:
        keep = O.dropout_keep(*dkeys, T, K, p)
        ks = O.dropout_scale(p)
    Y, U, Z = O.forward(X, W, A, B, s, keep, ks, mag, nrm)
    gr = O.backward(X, dY, W, A, B, s, U, keep, ks, mag, nrm, Z)
    return dict(Y=Y, U=U, Z=Z, **gr)


def _dora_vectors(got, c, s):
    """The oracle's DoRA magnitude (||W_i||) and detached norm (||W_i + s B_i A||)
    for case c; the GPU's own vectors (lora_dora_row_norms) must agree with
    them to 1e-5 before the oracle runs on its own."""
    W, A, B = np64(c["W"]), np64(c["A"]), np64(c["B"])
    mag, nrm = O.dora_row_norms(W), O.dora_row_norms(W, A, B, s)
    assert rel_err(got["mag"], mag) <= 1e-5
    assert rel_err(got["norm"], nrm) <= 1e-5
    return mag, nrm


def _check_full(got, ref, tol, dora, names=("Y", "U", "dX", "dA", "dB")):
    """Every output against the oracle, element by element over the whole
    tensor.  Y, dX (and Z) meet the path's bar; U, dA and dB are float32-exact
    on every path (rank-side products in float32); the DoRA magnitude gradient
    reads Z and so meets the path's bar."""
    for n in tuple(names) + (("Z", "dmag") if dora else ()):
        e = rel_err(got[n], ref[n])
        bar = 1e-4 if n in ("U", "dA", "dB") else tol
        _say(f"  {n}: rel err {e:.3e} (bar {bar:g})")
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten (NaN) elements"
        assert e <= bar, (n, e)


# ------------------------------------------------------------- dropout -----
@pytest.mark.parametrize("T,K,p,keys", [
    (33, 72, 0.05, (1234, 0, 0, 0, 0)),
    (128, 2048, 0.05, (1234, 3, 2, 21, 2)),
    (64, 2560, 0.1, (1235, 7, 1, 35, 6)),
    (1, 4, 0.5, (0, 0, 0, 0, 0)),
    (17, 9728, 0.1, (2**63 + 11, 2**40, 1, 5, 4)),
])
def test_dropout_mask_bit_exact(T, K, p, keys):
    _say("dropout", T, K, p, keys)
    mask = torch.full((T, K), 7, device=DEV, dtype=torch.uint8)
    L.lora_dropout_mask(L.make_dropout(*keys, p), T, K, mask)
    got = mask.cpu().numpy().astype(bool)
    ref = O.dropout_keep(*keys, T, K, p)
    assert np.array_equal(got, ref)


# ------------------------------------------------- per-linear fwd / bwd ----
LINEAR_CASES = [
    # name, T, K, N, r, w dtype, scale, dropout p, dora, x_std, dy_std
    ("single-64x64", 32, 64, 64, 4, "f32", 2.0, 0.0, False, 1.0, 1.0),
    ("ragged-f32", 37, 84, 100, 8, "f32", 2.0, 0.1, False, 1.0, 1.0),
    ("ragged-f32-dora", 37, 84, 100, 8, "f32", 1.5, 0.1, True, 1.0, 1.0),
    ("ragged-f32-r128", 70, 132, 136, 128, "f32", 0.5, 0.0, False, 1.0, 1.0),
    ("tinyllama-wq", 128, 2048, 2048, 8, "f32", 2.0, 0.05, False, 1.0, 1e-2),
    ("tinyllama-wv", 128, 2048, 256, 8, "f32", 2.0, 0.05, False, 1.0, 1e-2),
    ("wide-4096", 1536, 4096, 4096, 16, "f32", 2.0, 0.0, False, 1.0, 1.0),
    ("ragged-bf16", 70, 136, 264, 32, "bf16", math.sqrt(32), 0.1, False, 1.0, 1e-2),
    ("ragged-bf16-dora", 129, 264, 136, 64, "bf16", 1.0, 0.1, True, 1.0, 1e-2),
    ("qwen-wq-slice", 256, 2560, 4096, 32, "bf16", math.sqrt(32), 0.0, False, 1.0, 1e-2),
    ("qwen-wdown-slice", 256, 9728, 2560, 32, "bf16", math.sqrt(32), 0.0, False, 1.0, 1e-2),
    ("qwen-dora-wgate-slice", 256, 2560, 9728, 64, "bf16", 1.0, 0.1, True, 1.0, 1e-2),
    # short chunks: contraction split across blocks, rank-side work beside the GEMM
    ("split-ragged-f32", 100, 1000, 600, 8, "f32", 2.0, 0.1, False, 1.0, 1.0),
    ("split-ragged-f32-dora", 72, 1032, 520, 12, "f32", 1.5, 0.1, True, 1.0, 1.0),
    ("split-f32-r32", 128, 1024, 768, 32, "f32", 2.0, 0.05, False, 1.0, 1e-2),
    ("split-f32-token-ranges", 400, 1024, 512, 8, "f32", 2.0, 0.05, False, 1.0, 1.0),
    ("split-f32-v-reduced", 128, 1088, 8192, 32, "f32", 2.0, 0.05, False, 1.0, 1e-2),
    ("split-f32-r40", 128, 1024, 512, 40, "f32", 2.0, 0.1, False, 1.0, 1.0),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=[c[0] for c in LINEAR_CASES])
def test_linear_forward_backward_parity(case):
    name, T, K, N, r, wd, s, p, dora, xs, dys = case
    _say("linear", name)
    c = _linear_case(T, K, N, r, wd, seed=zlib.crc32(name.encode()) % 1000, x_std=xs, dy_std=dys)
    dk = (1234, 2, 1, 3, 4)
    got = _run_gpu(c, s, p, dk, dora)
    mag, nrm = _dora_vectors(got, c, s) if dora else (None, None)
    ref = _oracle(c, s, p, dk, mag, nrm)
    tol = TOL[wd]
    names = ["Y", "U", "dX", "dA", "dB"] + (["Z", "dmag"] if dora else [])
    for n in names:
        e = rel_err(got[n], ref[n])
        _say(f"  {n}: rel err {e:.3e}")
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten (NaN) elements"
        assert e <= tol, (n, e)


# The direct-operand bf16 loop (tile configuration 5: the activation operand
# in fragment tiles, loaded straight into registers; W through LDS).  Pinned
# so that small shapes take it; each product uses it where its contraction
# is a multiple of 64 (the forward's in_dim, the dX product's out_dim).
DIRECT_CASES = [
    # name, T, K, N, r, scale, dropout p, DoRA
    ("direct-fwd-ragged-tiles", 288, 640, 1000, 32, math.sqrt(32), 0.1, True),
    ("direct-dx-ragged-cols", 96, 600, 1088, 16, 2.0, 0.1, False),
    ("direct-split-contraction", 256, 2560, 512, 64, 1.0, 0.1, True),
    ("direct-whole-tiles", 512, 1024, 768, 64, 1.0, 0.0, False),
    ("direct-rank-128", 128, 640, 1088, 128, 1.0, 0.2, True),   # LoRA term in two rank chunks
]


@pytest.fixture
def bf16_config_5():
    L.lora_set_bf16_config(5)
    try:
        yield
    finally:
        L.lora_set_bf16_config(-1)


@pytest.mark.parametrize("case", DIRECT_CASES, ids=[c[0] for c in DIRECT_CASES])
def test_direct_operand_products_match_oracle(case, bf16_config_5):
    name, T, K, N, r, s, p, dora = case
    _say("direct", name)
    c = _linear_case(T, K, N, r, "bf16", seed=zlib.crc32(name.encode()) % 1000, dy_std=1e-2)
    dk = (1234, 2, 1, 3, 4)
    got = _run_gpu(c, s, p, dk, dora)
    mag, nrm = _dora_vectors(got, c, s) if dora else (None, None)
    ref = _oracle(c, s, p, dk, mag, nrm)
    for n in ["Y", "U", "dX", "dA", "dB"] + (["Z", "dmag"] if dora else []):
        e = rel_err(got[n], ref[n])
        _say(f"  {n}: rel err {e:.3e}")
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten (NaN) elements"
        assert e <= TOL["bf16"], (n, e)


QUANT_CASES = [
    # name, format, T, K, N, r, scale, dropout p (, DoRA)
    ("q8_0-ragged", "q8_0", 100, 544, 264, 8, 2.0, 0.1),
    ("q4_0-ragged", "q4_0", 300, 1056, 520, 16, 2.0, 0.1),
    ("q4_k-tiles", "q4_k", 256, 512, 264, 32, math.sqrt(32), 0.0),
    ("q6_k-ragged", "q6_k", 72, 768, 136, 8, 2.0, 0.1),
    ("q4_k-qwen-wq-slice", "q4_k", 256, 2560, 4096, 32, math.sqrt(32), 0.0),
    ("q6_k-qwen-wdown-slice", "q6_k", 256, 9728, 2560, 32, math.sqrt(32), 0.1),
    ("q4_0-split-k", "q4_0", 64, 4096, 512, 16, 2.0, 0.05),
    ("q4_k-dora", "q4_k", 129, 512, 264, 64, 1.0, 0.1, True),
    ("q6_k-dora-wdown-slice", "q6_k", 256, 9728, 2560, 64, 1.0, 0.1, True),
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quantized_w_forward_backward_parity(case):
    """Block-quantized frozen W against the oracle on the decoded weights,
    at the bf16 bar (the products run in bf16 on the decoded W)."""
    name, fmt, T, K, N, r, s, p = case[:8]
    dora = len(case) > 8 and case[8]
    _say("quantized linear", name)
    c = _linear_case(T, K, N, r, fmt, seed=zlib.crc32(name.encode()) % 1000, dy_std=1e-2)
    dk = (1234, 2, 1, 3, 4)
    got = _run_gpu(c, s, p, dk, dora)
    # the magnitude initialisation and the refresh over the decoded base
    mag, nrm = _dora_vectors(got, c, s) if dora else (None, None)
    ref = _oracle(c, s, p, dk, mag, nrm)
    for n in ("Y", "U", "dX", "dA", "dB") + (("Z", "dmag") if dora else ()):
        e = rel_err(got[n], ref[n])
        _say(f"  {n}: rel err {e:.3e}")
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten (NaN) elements"
        assert e <= TOL[fmt], (n, e)


@pytest.mark.parametrize("wd_,T,K,N", [("f32", 64, 256, 320), ("q4_k", 96, 512, 264), ("bf16", 96, 600, 1000)])
def test_pinned_direct_configuration_leaves_ineligible_products_alone(wd_, T, K, N, bf16_config_5):
    """With configuration 5 pinned, products it cannot run (float32 W, a
    quantized base, bf16 contractions that are not whole 64-wide K-steps:
    here both the forward's 600 and the dX product's 1000) keep the
    planner's choice and their results."""
    c = _linear_case(T, K, N, 16, wd_, seed=T + K, dy_std=1e-2)
    dk = (1234, 2, 1, 3, 4)
    got = _run_gpu(c, 2.0, 0.1, dk, False)
    ref = _oracle(c, 2.0, 0.1, dk, None, None)
    for n in ("Y", "U", "dX", "dA", "dB"):
        assert torch.isfinite(got[n]).all(), n
        assert rel_err(got[n], ref[n]) <= TOL[wd_], n


def _exact_planes(fmt, planes, seed):
    """Scales that make every decoded weight a bf16 value: powers of two and
    small sub-scales (and Q4_K's dmin equal to d, with mins below 16)."""
    g = torch.Generator().manual_seed(seed)
    pl = dict(planes)
    pow2 = lambda shape: (2.0 ** -torch.randint(6, 12, shape, generator=g)).to(torch.float16)
    if fmt in ("q8_0", "q4_0"):
        pl["d"] = pow2(planes["d"].shape)
    elif fmt == "q4_k":
        d = pow2(planes["dm"].shape[:2] + (1,))
        pl["dm"] = torch.cat([d, d], dim=2)
        sc = torch.randint(1, 8, planes["sm"].shape[:2] + (1,), generator=g).to(torch.uint8)
        mn = torch.randint(0, 16, planes["sm"].shape[:2] + (1,), generator=g).to(torch.uint8)
        pl["sm"] = torch.cat([sc, mn], dim=2)
    else:
        pl["d"] = pow2(planes["d"].shape)
        pl["sc"] = torch.randint(-3, 4, planes["sc"].shape, generator=g).to(torch.int8)
    return pl


@pytest.mark.parametrize("fmt,T,K,N", [("q8_0", 100, 544, 264), ("q4_0", 130, 1024, 520),
                                       ("q4_k", 256, 512, 264), ("q6_k", 72, 768, 136)])
def test_quantized_w_equals_bf16_w_when_exact(fmt, T, K, N):
    """When every decoded weight is a bf16 value, the quantized path stages
    bitwise the tiles the bf16 path stages: all outputs are equal."""
    r = 8
    _say("quantized vs bf16", fmt, T, K, N)
    c = _linear_case(T, K, N, r, fmt, seed=31)
    _, _, _, _, planes = c["Wq"]
    planes = _exact_planes(fmt, planes, 7)
    c["Wq"] = ("qweight", fmt, N, K, planes)
    W = Q.dequantize(fmt, {k: v.numpy() for k, v in planes.items()})
    Wb = torch.from_numpy(W).to(torch.bfloat16)
    assert np.array_equal(Wb.double().numpy(), W)
    cb = dict(c)
    cb["Wq"], cb["W"] = Wb, Wb.float()
    a = _run_gpu(c, 2.0, 0.1)
    b = _run_gpu(cb, 2.0, 0.1)
    for n in ("Y", "U", "dX", "dA", "dB"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("T,K,N,r", [(64, 128, 96, 8), (128, 1024, 512, 8)])
def test_backward_accumulates_over_chunks(T, K, N, r):
    c1 = _linear_case(T, K, N, r, seed=1)
    c2 = dict(c1)
    c2["X"] = WL.draw((T, K), (77, 0, 0, 0, 1, "X"), "normal", 1.0)
    c2["dY"] = WL.draw((T, N), (77, 0, 0, 0, 1, "dY"), "normal", 1.0)
    g1, g2 = _gpu(c1), _gpu(c2)
    lin = L.make_linear(g1["Wq"], g1["A"], g1["B"], 2.0, T)
    ws = torch.empty(L.lora_workspace_bytes(lin), device=DEV, dtype=torch.uint8)
    dA = torch.full((r, K), float("nan"), device=DEV)
    dB = torch.full((N, r), float("nan"), device=DEV)
    for i, g in enumerate((g1, g2)):
        Y = torch.empty(T, N, device=DEV)
        U = torch.empty(T, r, device=DEV)
        L.lora_forward(lin, g["X"], Y, U, None, None, ws)
        L.lora_backward(lin, g["X"], g["dY"], U, None, None, dA, dB, None, i > 0, None, ws)
    r1, r2 = _oracle(c1, 2.0), _oracle(c2, 2.0)
    assert rel_err(dA, r1["dA"] + r2["dA"]) <= 1e-4
    assert rel_err(dB, r1["dB"] + r2["dB"]) <= 1e-4


def test_zero_adapter_gives_exact_zero_dA_and_frozen_output():
    T, K, N, r = 96, 256, 192, 16
    c = _linear_case(T, K, N, r, seed=5)
    c["B"] = torch.zeros_like(c["B"])
    got = _run_gpu(c, 2.0, 0.1)
    assert torch.count_nonzero(got["dA"]).item() == 0
    frozen = np64(c["X"]) @ np64(c["W"]).T
    assert rel_err(got["Y"], frozen) <= 1e-5


def test_adjointness_of_frozen_products_on_gpu():
    """<X W^T, V> == <X, V W>: pins the native-layout dX GEMM to the forward."""
    T, K, N, r = 160, 384, 320, 8
    c = _linear_case(T, K, N, r, seed=6)
    c["B"] = torch.zeros_like(c["B"])
    got = _run_gpu(c, 1.0)
    lhs = float((np64(got["Y"]) * np64(c["dY"])).sum())
    rhs = float((np64(c["X"]) * np64(got["dX"])).sum())
    assert abs(lhs - rhs) <= 1e-5 * (np.abs(np64(got["Y"])).sum() + 1.0)


def test_linear_outputs_are_deterministic():
    c = _linear_case(200, 512, 384, 16, seed=7)
    a = _run_gpu(c, 2.0, 0.1)
    b = _run_gpu(c, 2.0, 0.1)
    for n in ("Y", "U", "dX", "dA", "dB"):
        assert torch.equal(a[n], b[n]), n


# ------------------------------------------------ full-size, every output --
FULL_CASES = [
    # workload, projection index: the launch plans the bench times, including
    # split-contraction bf16 products in both directions.  Every projection
    # shape of the Qwen3-4B-shaped layers at 4096 tokens, and the DoRA
    # workload's shapes at 2048 tokens.
    (4, 0), (4, 1), (4, 3), (4, 4), (4, 6), (5, 0), (5, 2), (5, 3), (5, 4), (5, 6),
]


@pytest.mark.parametrize("wl,pi", FULL_CASES, ids=[f"wl{a}-p{b}" for a, b in FULL_CASES])
def test_full_size_linear(wl, pi):
    """Full workload shape in the launch plan the bench uses; every output
    against the oracle's forward and backward on the same full inputs."""
    cfg = WL.get_config(wl)
    proj = cfg.projections[pi]
    _say("full-size", cfg.name, proj.name)
    inp = WL.linear_inputs(cfg, 0, proj, device=DEV, chunks=1)
    s = O.scaling(cfg.alpha, cfg.rank, cfg.scaling)
    c = {"Wq": inp.get("W_bf16", inp["W"]), "W": inp["W"], "A": inp["A"], "B": inp["B"],
         "X": inp["X"][0], "dY": inp["dY"][0]}
    p = cfg.dropout
    dk = (cfg.seeds[0], 0, 0, 0, proj.ordinal)
    got = _run_gpu(c, s, p, dk, cfg.dora)
    mag, nrm = _dora_vectors(got, c, s) if cfg.dora else (None, None)
    ref = _oracle(c, s, p, dk, mag, nrm)
    _check_full(got, ref, TOL[cfg.w_dtype], cfg.dora)


@pytest.mark.parametrize("pi,from_y", [(4, False), (6, False), (4, True), (0, True), (1, True)],
                         ids=["wgate", "wdown", "wgate-from-y", "wq-from-y", "wk-from-y"])
def test_full_size_stacked_slots(pi, from_y):
    """The DoRA workload's two slots at full size in the launch plan the
    bench times (one product over both slots' 2 x 2048 stacked rows per
    direction); each slot against the oracle over every output.  from_y:
    as the trainer runs it, the forward writes Y only and the backward's
    magnitude gradient reads Y."""
    cfg = WL.get_config(5)
    proj = cfg.projections[pi]
    _say("full-size stacked slots", cfg.name, proj.name)
    s = O.scaling(cfg.alpha, cfg.rank, cfg.scaling)
    T, N = cfg.tokens, proj.out_dim
    cs = []
    for si in range(2):
        inp = WL.linear_inputs(cfg, 0, proj, slot=si, device=DEV, chunks=1)
        cs.append({"Wq": inp["W_bf16"], "W": inp["W"], "A": inp["A"], "B": inp["B"],
                   "X": inp["X"][0], "dY": inp["dY"][0]})
    cs[1]["Wq"], cs[1]["W"] = cs[0]["Wq"], cs[0]["W"]
    # seeded magnitudes away from ||W|| (an input, like A and B)
    mags = [WL.draw((N,), (5, i, 0, proj.ordinal, 0, "B"), "uniform", 0.5, DEV) + 1.0
            for i in range(2)]
    nrms = [torch.empty(N, device=DEV) for _ in cs]
    for c, n in zip(cs, nrms):
        L.lora_dora_row_norms(L.make_linear(c["Wq"], c["A"], c["B"], s, T), n)
    lins = [L.make_linear(c["Wq"], c["A"], c["B"], s, T, m, n, dora_from_y=from_y)
            for c, m, n in zip(cs, mags, nrms)]
    shapes = dict(Y=(T, N), U=(T, cfg.rank), dX=(T, proj.in_dim), dA=(cfg.rank, proj.in_dim),
                  dB=(N, cfg.rank), Z=(T, N), dmag=(N,))
    out = {k: [torch.full(v, float("nan"), device=DEV) for _ in cs] for k, v in shapes.items()}
    ws = torch.empty(L.lora_slots_workspace_bytes(lins), device=DEV, dtype=torch.uint8)
    dks = [(cfg.seeds[i], 0, 0, 0, proj.ordinal) for i in range(2)]
    drops = [L.make_dropout(*k, cfg.dropout) for k in dks]
    L.lora_forward_slots(lins, [c["X"] for c in cs], out["Y"], out["U"],
                         None if from_y else out["Z"], drops, ws)
    L.lora_backward_slots(lins, [c["X"] for c in cs], [c["dY"] for c in cs], out["U"],
                          out["Y"] if from_y else out["Z"],
                          out["dX"], out["dA"], out["dB"], out["dmag"], drops=drops, ws=ws)
    torch.cuda.synchronize()
    for i, c in enumerate(cs):
        got = {k: v[i] for k, v in out.items()}
        nrm = O.dora_row_norms(np64(c["W"]), np64(c["A"]), np64(c["B"]), s)
        assert rel_err(nrms[i], nrm) <= 1e-5
        ref = _oracle(c, s, cfg.dropout, dks[i], np64(mags[i]), nrm)
        if from_y:
            assert torch.isnan(got["Z"]).all(), "the forward wrote Z"
            _check_full(got, ref, TOL["bf16"], False, names=("Y", "U", "dX", "dA", "dB", "dmag"))
        else:
            _check_full(got, ref, TOL["bf16"], True)


@pytest.mark.parametrize("fmt,pi", [("q4_k", 4), ("q6_k", 6), ("q8_0", 0)],
                         ids=["q4_k-wgate", "q6_k-wdown", "q8_0-wq"])
def test_full_size_quantized(fmt, pi):
    """Qwen3-4B-shaped projection at its full 4096 tokens over a quantized
    base, in the launch plan the bench's --w-format runs use; every output
    against the oracle on the decoded weights."""
    cfg = WL.get_config(4)
    proj = cfg.projections[pi]
    _say("full-size quantized", fmt, proj.name)
    s = O.scaling(cfg.alpha, cfg.rank, cfg.scaling)
    N, K, T = proj.out_dim, proj.in_dim, cfg.tokens
    inp = WL.linear_inputs(cfg, 0, proj, device=DEV, chunks=1)
    planes = WL.qweight_planes(fmt, N, K, (cfg.number, 0, 0, proj.ordinal), device=DEV)
    c = {"Wq": L.qweight_pack(fmt, N, K, planes),
         "W": torch.from_numpy(Q.dequantize(fmt, {k: v.cpu().numpy() for k, v in planes.items()})),
         "A": inp["A"], "B": inp["B"], "X": inp["X"][0], "dY": inp["dY"][0]}
    lin = L.make_linear(c["Wq"], c["A"], c["B"], s, T)
    got = {k: torch.full(v, float("nan"), device=DEV) for k, v in
           dict(Y=(T, N), U=(T, cfg.rank), dX=(T, K), dA=(cfg.rank, K), dB=(N, cfg.rank)).items()}
    ws = torch.empty(L.lora_workspace_bytes(lin), device=DEV, dtype=torch.uint8)
    L.lora_forward(lin, c["X"], got["Y"], got["U"], None, None, ws)
    L.lora_backward(lin, c["X"], c["dY"], got["U"], None, got["dX"], got["dA"], got["dB"], ws=ws)
    torch.cuda.synchronize()
    _check_full(got, _oracle(c, s), TOL[fmt], False)


# --------------------------------------------------- prepare and AdamW -----
@pytest.mark.parametrize("n,scale,max_norm,n_pred", [
    (1, 3.0, 1.0, 1), (1003, 10.0, 1.0, 4), (131072, 1e-3, 1.0, 1536), (1126400, 1.0, 0.0, 512),
    (5_000_001, 0.5, 2.0, 8),
])
def test_grad_prepare_parity(n, scale, max_norm, n_pred):
    g = WL.draw((n,), (500, 0, 0, 0, n % 97, "dY"), "normal", scale)
    gd = g.to(DEV)
    d_scale = torch.zeros(1, device=DEV)
    stats = torch.zeros(2, device=DEV, dtype=torch.float64)
    ws = torch.empty(L.lora_grad_prepare_workspace_bytes(n), device=DEV, dtype=torch.uint8)
    norm = L.lora_grad_prepare(gd, n_pred, max_norm, d_scale, stats, True, ws)
    ref = O.grad_prepare([np64(g)], n_pred, max_norm)
    assert norm == pytest.approx(ref["norm"], rel=1e-12)
    assert d_scale.item() == pytest.approx(ref["scale"], rel=1e-6)
    assert stats[1].item() == pytest.approx(ref["clip"], rel=1e-12)
    if ref["clip"] < 1.0:   # clipped: the prepared gradient has norm max_norm
        assert np.linalg.norm(np64(g) * d_scale.item()) == pytest.approx(max_norm, rel=1e-6)


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), -float("inf")])
def test_grad_prepare_vetoes_non_finite(bad):
    g = torch.randn(10000, device=DEV)
    g[1234] = bad
    d_scale = torch.zeros(1, device=DEV)
    ws = torch.empty(L.lora_grad_prepare_workspace_bytes(g.numel()), device=DEV, dtype=torch.uint8)
    with pytest.raises(L.LoraError) as e:
        L.lora_grad_prepare(g, 4, 1.0, d_scale, None, True, ws)
    assert e.value.status == L.LORA_E_NONFINITE
    assert math.isnan(d_scale.item())
    # AdamW on a vetoed scale changes nothing
    p = torch.randn(10000, device=DEV)
    m = torch.randn(10000, device=DEV)
    v = torch.rand(10000, device=DEV)
    before = [x.clone() for x in (p, m, v)]
    L.lora_adamw_step(p, torch.nan_to_num(g), m, v, [(0, 10000, 0)],
                      L.LoraAdamwHparams(1e-3, 0.9, 0.999, 1e-8, 0.1, 1.0, 3), d_scale)
    for x, y in zip((p, m, v), before):
        assert torch.equal(x, y)


@pytest.mark.parametrize("t", [1, 2, 7])
def test_adamw_parity_on_shared_inputs(t):
    segs = [(0, 4096, 0), (4096, 1000, 1), (5096, 2000, 2), (7096, 4, 0)]
    n = 7100
    p0 = WL.draw((n,), (501, t, 0, 0, 0, "A"), "normal", 0.05)
    g0 = WL.draw((n,), (501, t, 0, 0, 0, "dY"), "normal", 1.0)
    m0 = WL.draw((n,), (501, t, 0, 0, 0, "X"), "normal", 0.01) * (t > 1)
    v0 = WL.draw((n,), (501, t, 0, 0, 0, "B"), "uniform", 1e-4).abs() * (t > 1)
    c = float(np.float32(0.125))
    lr, wd, ratio = 2e-4, 0.1, 16.0
    P, G, M, V = (x.to(DEV) for x in (p0, g0, m0, v0))
    d_scale = torch.tensor([c], device=DEV)
    L.lora_adamw_step(P, G, M, V, segs, L.LoraAdamwHparams(lr, 0.9, 0.999, 1e-8, wd, ratio, t), d_scale)
    kinds = {0: "A", 1: "B", 2: "mag"}
    for off, cnt, kind in segs:
        sl = slice(off, off + cnt)
        pr, mr, vr = O.adamw_update(np64(p0[sl]), np64(g0[sl]), np64(m0[sl]), np64(v0[sl]),
                                    kinds[kind], lr, t, c, weight_decay=wd, plus_ratio=ratio)
        assert rel_err(np64(P[sl]) - np64(p0[sl]), pr - np64(p0[sl])) <= 1e-4
        assert rel_err(M[sl], mr) <= 1e-5
        assert rel_err(V[sl], vr) <= 1e-5


def _arena_segments(cfg):
    """Sizes of a slot's arena segments [all A | all B | all DoRA magnitudes]
    over every layer and projection of a workload."""
    na = cfg.layers * sum(cfg.rank * p.in_dim for p in cfg.projections)
    nb = cfg.layers * sum(p.out_dim * cfg.rank for p in cfg.projections)
    nm = cfg.layers * sum(p.out_dim for p in cfg.projections) if cfg.dora else 0
    segs = [(0, na, L.KIND_A), (na, nb, L.KIND_B)] + ([(na + nb, nm, L.KIND_MAG)] if nm else [])
    return na + nb + nm, segs


@pytest.mark.parametrize("wl,n_expect", [(4, 66_060_288), (5, 133_226_496)])
def test_prepare_and_adamw_on_the_full_arena(wl, n_expect):
    """Gradient preparation and AdamW over a whole slot's arena at the
    workload's size (all 36 layers x 7 projections: the clip norm is global
    over it), against the oracle's grad_prepare and adamw_update on the same
    values.  Third update of the slot (nonzero moments), the workload's
    hyper-parameters; the arena's gradient is scaled so that the clip acts."""
    cfg = WL.get_config(wl)
    n, segs = _arena_segments(cfg)
    assert n == n_expect
    _say("full arena", cfg.name, n)
    key = lambda kind: (600 + wl, 0, 0, 0, 3, kind)
    g = WL.draw((n,), key("dY"), "normal", 2.0, DEV)   # norm/Npred about 3: the clip acts
    p0 = WL.draw((n,), key("A"), "normal", 0.02, DEV)
    m0 = WL.draw((n,), key("X"), "normal", 1e-4, DEV)
    v0 = WL.draw((n,), key("B"), "uniform", 1e-8, DEV).abs_()
    P, M, V = p0.clone(), m0.clone(), v0.clone()
    n_pred = cfg.tokens * cfg.chunks
    d_scale = torch.zeros(1, device=DEV)
    stats = torch.zeros(2, device=DEV, dtype=torch.float64)
    ws = torch.empty(L.lora_grad_prepare_workspace_bytes(n), device=DEV, dtype=torch.uint8)
    norm = L.lora_grad_prepare(g, n_pred, cfg.max_norm, d_scale, stats, True, ws)
    t, lr = 3, O.lr_at(2, cfg.lr, cfg.schedule, cfg.warmup, cfg.total_updates, cfg.lr_min)
    L.lora_adamw_step(P, g, M, V, segs,
                      L.LoraAdamwHparams(lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay,
                                         cfg.plus_ratio, t), d_scale)
    torch.cuda.synchronize()
    gh = np64(g)
    ref = O.grad_prepare([gh], n_pred, cfg.max_norm)
    assert ref["clip"] < 1.0   # the clip acts at this scale
    assert norm == pytest.approx(ref["norm"], rel=1e-12)
    assert stats[1].item() == pytest.approx(ref["clip"], rel=1e-12)
    assert d_scale.item() == pytest.approx(ref["scale"], rel=1e-6)
    kinds = {L.KIND_A: "A", L.KIND_B: "B", L.KIND_MAG: "mag"}
    Ph, Mh, Vh, p0h, m0h, v0h = (np64(x) for x in (P, M, V, p0, m0, v0))
    for off, cnt, kind in segs:
        for c0 in range(off, off + cnt, 1 << 24):   # bounded host memory
            sl = slice(c0, min(off + cnt, c0 + (1 << 24)))
            pr, mr, vr = O.adamw_update(p0h[sl], gh[sl], m0h[sl], v0h[sl], kinds[kind], lr, t,
                                        ref["scale"], cfg.beta1, cfg.beta2, cfg.eps,
                                        cfg.weight_decay, cfg.plus_ratio)
            assert rel_err(Ph[sl] - p0h[sl], pr - p0h[sl]) <= 1e-4, (kind, c0)
            assert rel_err(Mh[sl], mr) <= 1e-5, (kind, c0)
            assert rel_err(Vh[sl], vr) <= 1e-5, (kind, c0)


@pytest.mark.parametrize("split", [True, False], ids=["split", "whole-rows"])
@pytest.mark.parametrize("wd_,N,K,r", [
    ("f32", 100, 84, 8),          # ragged rows and a partial last chunk
    ("bf16", 264, 136, 64),
    ("bf16", 45, 100, 12),        # rows not 16-byte aligned: element loads
    ("f32", 33, 4097, 128),       # rank 128, odd K, many column splits
    ("bf16", 2560, 9728, 64),     # DoRA workload shapes (wdown, wup)
    ("bf16", 9728, 2560, 64),
    ("f32", 2048, 2048, 8),
    ("q4_k", 264, 512, 32),       # quantized bases: decoded to float32 in the pass
    ("q6_k", 136, 768, 64),
    ("q4_0", 100, 1056, 8),       # ragged rows, a half last chunk
    ("q8_0", 45, 544, 12),
    ("q4_k", 2560, 9728, 64),
])
def test_dora_row_norms_parity(wd_, N, K, r, split):
    c = _linear_case(8, K, N, r, wd_, seed=11, b_std=0.05)
    g = _gpu(c)
    out = torch.full((N,), float("nan"), device=DEV)
    L.lora_dora_row_norms(L.make_linear(g["Wq"], None, None, 1.0, 8), out, split=split)
    assert rel_err(out, O.dora_row_norms(np64(c["W"]))) <= 1e-5
    out.fill_(float("nan"))
    L.lora_dora_row_norms(L.make_linear(g["Wq"], g["A"], g["B"], 1.7, 8), out, split=split)
    assert rel_err(out, O.dora_row_norms(np64(c["W"]), np64(c["A"]), np64(c["B"]), 1.7)) <= 1e-5


def test_dora_row_norms_workspace_checked():
    c = _linear_case(8, 9728, 64, 16, "bf16", seed=3)
    g = _gpu(c)
    lin = L.make_linear(g["Wq"], g["A"], g["B"], 1.0, 8)
    need = L.lora_dora_row_norms_workspace_bytes(lin)
    assert need > 0
    out = torch.empty(64, device=DEV)
    with pytest.raises(L.LoraError):
        L.lora_dora_row_norms(lin, out, torch.empty(need - 8, device=DEV, dtype=torch.uint8))


def _slot_factors(K, N, r, slots, seed, b_std):
    """Per-slot A and B over one W (the adapters of one base)."""
    out = []
    for q in range(slots):
        key = lambda kind: (950 + seed, q, 0, 0, 0, kind)
        out.append((WL.draw((r, K), key("A"), "uniform", 1 / math.sqrt(K)),
                    WL.draw((N, r), key("B"), "normal", b_std)))
    return out


# (N, K, r, slots, b_std): ragged rows and K (K % 32 != 0), ranks padded to
# 32 or 64, four slots (two column tiles), long K (contraction splits), a
# LoRA term as large as W (b_std 1.0), the DoRA workload's shapes.
BATCH_CASES = [
    (100, 136, 8, 1, 0.05),
    (37, 1000, 40, 2, 1.0),
    (264, 520, 64, 4, 0.5),
    (300, 7000, 16, 3, 1.0),
    (129, 2048, 64, 2, 0.05),
    (9728, 2560, 64, 2, 0.05),
    (2560, 9728, 64, 2, 0.05),
]


@pytest.mark.parametrize("N,K,r,slots,b_std", BATCH_CASES,
                         ids=[f"{c[0]}x{c[1]}-r{c[2]}-s{c[3]}" for c in BATCH_CASES])
def test_dora_row_norms_batch_parity(N, K, r, slots, b_std):
    """The expansion over bf16 W (slots stacked over one pass of W) against
    the oracle's norms of the formed rows."""
    W = WL.draw((N, K), (960, 0, 0, 0, 0, "W"), "normal", 0.02).to(torch.bfloat16)
    fac = _slot_factors(K, N, r, slots, 1, b_std)
    Wd = W.to(DEV)
    dev = [(A.to(DEV), B.to(DEV)) for A, B in fac]
    scales = [1.7 + 0.3 * q for q in range(slots)]
    lins = [L.make_linear(Wd, A, B, s, 8) for (A, B), s in zip(dev, scales)]
    outs = [torch.full((N,), float("nan"), device=DEV) for _ in range(slots)]
    L.lora_dora_row_norms_batch(lins, outs)
    Wh = np64(W.float())
    for q, ((A, B), s) in enumerate(zip(fac, scales)):
        assert rel_err(outs[q], O.dora_row_norms(Wh, np64(A), np64(B), s)) <= 1e-5, q


def test_dora_row_norms_batch_mixed_list():
    """Linears the expansion does not take (float32 or quantized W, rank
    above 64, no factors) run as lora_dora_row_norms, bitwise, in a list that
    also holds more W matrices than one launch takes (chunked launches)."""
    lins, outs, refs, direct = [], [], [], []
    keep = []
    for i in range(11):
        wd = ["bf16", "f32", "q4_k", "bf16"][i % 4] if i < 8 else "bf16"
        N, K = 64 + 40 * i, 512 if wd == "q4_k" else 256 + 72 * (i % 3)
        r = 128 if i == 3 else 8 + 8 * (i % 4)
        c = _linear_case(8, K, N, r, wd, seed=40 + i, b_std=0.3)
        g = _gpu(c)
        keep.append(g)
        bare = i == 7
        lin = L.make_linear(g["Wq"], None if bare else g["A"], None if bare else g["B"],
                            1.3, 8)
        lins.append(lin)
        outs.append(torch.full((N,), float("nan"), device=DEV))
        refs.append(O.dora_row_norms(np64(c["W"])) if bare else
                    O.dora_row_norms(np64(c["W"]), np64(c["A"]), np64(c["B"]), 1.3))
        direct.append(wd != "bf16" or r > 64 or bare)
    L.lora_dora_row_norms_batch(lins, outs)
    for i, (lin, out, ref) in enumerate(zip(lins, outs, refs)):
        assert rel_err(out, ref) <= 1e-5, i
        if direct[i]:
            one = torch.empty_like(out)
            L.lora_dora_row_norms(lin, one)
            assert torch.equal(out, one), i


def test_dora_row_norms_batch_checks():
    c = _linear_case(8, 512, 300, 16, "bf16", seed=5)
    g = _gpu(c)
    lins = [L.make_linear(g["Wq"], g["A"], g["B"], 1.0, 8)] * 2
    outs = [torch.empty(300, device=DEV) for _ in range(2)]
    need = L.lora_dora_row_norms_batch_workspace_bytes(lins)
    assert need > 0
    with pytest.raises(L.LoraError):
        L.lora_dora_row_norms_batch(lins, outs, torch.empty(need - 256, device=DEV,
                                                            dtype=torch.uint8))
    bad = L.make_linear(g["Wq"], g["A"], g["B"], 1.0, 8)
    bad.rank = 200
    with pytest.raises(L.LoraError):
        L.lora_dora_row_norms_batch([lins[0], bad], outs)
    # Repeated calls give the same bits (fixed-order sums, no atomics).
    ws = torch.empty(need, device=DEV, dtype=torch.uint8)
    L.lora_dora_row_norms_batch(lins, outs, ws)
    first = [o.clone() for o in outs]
    ws.fill_(7)
    L.lora_dora_row_norms_batch(lins, outs, ws)
    assert all(torch.equal(a, b) for a, b in zip(first, outs))


# ------------------------------------------------------ end-to-end steps ---
def _e2e(cfg, layers=None, tokens=None, steps=1, slots=None, together=False):
    """Run `steps` updates on the GPU and in the oracle from equal inputs;
    return both states and gradients.  together: all slots step through the
    trainer's stacked slot path."""
    layers = cfg.layers if layers is None else layers
    T = cfg.tokens if tokens is None else tokens
    nslots = cfg.slots if slots is None else slots
    s = O.scaling(cfg.alpha, cfg.rank, cfg.scaling)
    W, Wq = {}, {}
    for l in range(layers):
        for pj in cfg.projections:
            inp = WL.linear_inputs(cfg, l, pj, chunks=0, tokens=T)
            W[(l, pj.ordinal)] = inp["W"]
            Wq[(l, pj.ordinal)] = inp.get("W_bf16", inp["W"])
    model = S.FrozenModel(cfg, {k: v.to(DEV) for k, v in Wq.items()})
    trainer = S.Trainer(cfg, model, tokens=T, slots=nslots if together else 1)
    results = []
    staged = []
    for si in range(nslots):
        A, B, chunks = {}, {}, [dict() for _ in range(cfg.chunks)]
        for l in range(layers):
            for pj in cfg.projections:
                inp = WL.linear_inputs(cfg, l, pj, slot=si, tokens=T)
                key = (l, pj.ordinal)
                A[key], B[key] = inp["A"], inp["B"]
                for g in range(cfg.chunks):
                    chunks[g][key] = (inp["X"][g], inp["dY"][g])
        slot = S.Slot(cfg, model, {k: v.to(DEV) for k, v in A.items()},
                      {k: v.to(DEV) for k, v in B.items()}, cfg.seeds[si])
        if cfg.dora:
            trainer.init_dora(slot)
        ost = O.SlotState(params={k: {"A": np64(A[k]), "B": np64(B[k])} for k in A})
        if cfg.dora:
            for k in A:
                # the oracle's own ||W_i||; the GPU's initialisation must agree
                ost.params[k]["mag"] = O.dora_row_norms(np64(W[k]))
                assert rel_err(slot.mag[k], ost.params[k]["mag"]) <= 1e-5
                ost.norms[k] = O.dora_row_norms(np64(W[k]), ost.params[k]["A"], ost.params[k]["B"], s)
                assert rel_err(slot.norm[k], ost.norms[k]) <= 1e-5
        gchunks = [{k: (x.to(DEV), d.to(DEV)) for k, (x, d) in ch.items()} for ch in chunks]
        ochunks = [{k: (np64(x), np64(d)) for k, (x, d) in ch.items()} for ch in chunks]
        staged.append((si, slot, ost, gchunks, ochunks, []))
    lin64 = {k: np64(v) for k, v in W.items()}
    for it in range(steps):
        before = [(slot.params.clone(), {k: {n: a.copy() for n, a in v.items()}
                                          for k, v in ost.params.items()})
                  for _, slot, ost, _, _, _ in staged]
        if together:
            sts = trainer.step_slots([x[1] for x in staged], [x[3] for x in staged])
        else:
            sts = [trainer.step(slot, gch) for _, slot, _, gch, _, _ in staged]
        for (si, slot, ost, gch, och, hist), (p_before, o_before), st in zip(staged, before, sts):
            hp = dict(s=s, p=cfg.dropout, seed=cfg.seeds[si], n_pred=T * cfg.chunks,
                      max_norm=cfg.max_norm,
                      lr=O.lr_at(ost.k, cfg.lr, cfg.schedule, cfg.warmup, cfg.total_updates, cfg.lr_min),
                      weight_decay=cfg.weight_decay, plus_ratio=cfg.plus_ratio, dora=cfg.dora)
            res = O.train_step(ost, lin64, och, hp)
            hist.append((p_before, o_before, st, res, slot.grads.clone()))
    torch.cuda.synchronize()
    return [(slot, ost, hist) for _, slot, ost, _, _, hist in staged]


def _flat(slot, per_key, order=("A", "B", "mag")):
    """Oracle per-linear dict -> the slot arena order [A..., B..., mag...]."""
    parts = []
    for n in order:
        for k in slot.keys:
            if n in per_key[k]:
                parts.append(np.asarray(per_key[k][n], dtype=np.float64).ravel())
    return np.concatenate(parts)


E2E = [
    ("wl1", 1, None, None, 3, False),
    ("wl2", 2, None, None, 1, False),
    ("wl3", 3, None, None, 1, False),
    ("wl4-1layer-T512", 4, 1, 512, 2, False),
    ("wl5-1layer-T256", 5, 1, 256, 2, False),
    ("wl5-1layer-T256-stacked-slots", 5, 1, 256, 2, True),
    # real shapes: one full layer (all 7 projections) at the workloads' own
    # token counts, in the launch plans the bench times
    ("wl4-1layer-T4096", 4, 1, None, 2, False),
    ("wl5-1layer-2slots-2x2048-stacked", 5, 1, None, 2, True),
]


def _update_floor(e_grad, bar):
    """Smallest |g_ref| / max|g_ref| at which an element's update is compared.

    Adam divides each moment by its own root mean square, so an element's
    update moves with its gradient's error relative to that element, not to
    the segment's largest gradient; at t = 1 it is about -lr*sign(g).  An
    element whose reference gradient is at least e_grad/bar of the segment's
    largest has a relative gradient error of at most `bar` (e_grad being the
    measured max|g_gpu - g_ref| / max|g_ref| of the segment over all steps),
    so its update must meet `bar`.  Never below 1e-3 of the largest gradient
    (the exclusion the comparison reading starts from)."""
    return max(1e-3, e_grad / bar)


@pytest.mark.parametrize("name,wl,layers,tokens,steps,together", E2E, ids=[e[0] for e in E2E])
def test_end_to_end_step_parity(name, wl, layers, tokens, steps, together):
    """Whole updates against the oracle's train_step.

    Gradients: A and B are float32-exact on every path (rank-side products
    run in float32), so they meet 1e-4; the DoRA magnitude gradient reads Z,
    which a bf16-W frozen product rounds, so it meets the bf16 bar, and after
    a DoRA update the magnitude (trained on that gradient) scales every later
    gradient, so from the second step on a bf16 DoRA slot meets the bf16 bar
    throughout.  Updates meet the bar of their segment's gradients (1e-4 for
    float32-exact ones, 2e-2 for bf16-affected ones), compared where every
    step's reference gradient exceeds _update_floor of the segment's largest."""
    cfg = WL.get_config(wl)
    _say("e2e", name)
    for slot, ost, hist in _e2e(cfg, layers, tokens, steps, together=together):
        seg = {}
        for off, cnt, kind in slot.segments:
            seg[kind] = slice(off, off + cnt)
        e_grad = {kind: 0.0 for kind in seg}
        bf_seg = {kind: False for kind in seg}
        g_refs = []
        for it, (p_before, o_before, st, res, grads) in enumerate(hist):
            assert not st.vetoed and not res["vetoed"]
            assert st.norm == pytest.approx(res["prep"]["norm"], rel=1e-4)
            g_ref = _flat(slot, res["grads"])
            g_refs.append(g_ref)
            g_gpu = np64(grads)
            for kind, sl in seg.items():
                e = rel_err(g_gpu[sl], g_ref[sl])
                bf_dora = cfg.dora and cfg.w_dtype == "bf16"
                bf_hit = (kind == L.KIND_MAG and cfg.w_dtype == "bf16") or (bf_dora and it > 0)
                bar = TOL[cfg.w_dtype] if bf_hit else 1e-4
                bf_seg[kind] |= bf_hit
                e_grad[kind] = max(e_grad[kind], e)
                _say(f"  step {it} seg {kind}: grad rel err {e:.3e} (bar {bar:g})")
                assert e <= bar, (it, kind, e)
        p_before, o_before, st, res, grads = hist[-1]
        d_ref = _flat(slot, {k: {n: ost.params[k][n] - o_before[k][n] for n in ost.params[k]}
                             for k in ost.params})
        d_gpu = np64(slot.params) - np64(p_before)
        for kind, sl in seg.items():
            bar = 2e-2 if bf_seg[kind] else 1e-4
            floor = _update_floor(e_grad[kind], bar)
            m = np.ones(sl.stop - sl.start, dtype=bool)
            for g_ref in g_refs:
                m &= np.abs(g_ref[sl]) >= floor * np.abs(g_ref[sl]).max()
            e = rel_err(d_gpu[sl][m], d_ref[sl][m])
            _say(f"  update seg {kind}: rel err {e:.3e} (bar {bar:g}) over {m.sum()} of {m.size}"
                 f" (floor {floor:.2e})")
            assert m.sum() >= 0.25 * m.size, (kind, "too few elements compared")
            assert e <= bar, (kind, e)


def test_seeded_runs_give_identical_adapters():
    cfg = WL.get_config(2)
    digests = []
    for _ in range(2):
        (slot, _, _), = _e2e(cfg, layers=2, tokens=64, steps=2)
        digests.append(hashlib.sha256(slot.params.cpu().numpy().tobytes()).hexdigest())
    assert digests[0] == digests[1]


def _stream_inputs(cfg, layers, tokens):
    """Frozen W, and per slot A, B and chunks, on the GPU (seeded)."""
    Wq, per_slot = {}, []
    for l in range(layers):
        for pj in cfg.projections:
            inp = WL.linear_inputs(cfg, l, pj, chunks=0, tokens=tokens)
            Wq[(l, pj.ordinal)] = inp.get("W_bf16", inp["W"]).to(DEV)
    for si in range(cfg.slots):
        a, b, ch = {}, {}, [dict() for _ in range(cfg.chunks)]
        for l in range(layers):
            for pj in cfg.projections:
                inp = WL.linear_inputs(cfg, l, pj, slot=si, tokens=tokens)
                key = (l, pj.ordinal)
                a[key], b[key] = inp["A"].to(DEV), inp["B"].to(DEV)
                for g in range(cfg.chunks):
                    ch[g][key] = (inp["X"][g].to(DEV), inp["dY"][g].to(DEV))
        per_slot.append((a, b, ch))
    return Wq, per_slot


def _trained(cfg, inputs, tokens, steps, streams, together):
    """Adapters and gradients after `steps` updates of every slot through a
    trainer that spreads its calls over `streams` streams."""
    Wq, per_slot = inputs
    model = S.FrozenModel(cfg, Wq)
    trainer = S.Trainer(cfg, model, tokens=tokens, slots=cfg.slots if together else 1,
                        streams=streams)
    slots = []
    for si, (a, b, _) in enumerate(per_slot):
        slot = S.Slot(cfg, model, a, b, cfg.seeds[si])
        if cfg.dora:
            trainer.init_dora(slot)
        slots.append(slot)
    chunks = [ch for _, _, ch in per_slot]
    for _ in range(steps):
        if together:
            trainer.step_slots(slots, chunks)
        else:
            for slot, ch in zip(slots, chunks):
                trainer.step(slot, ch)
    torch.cuda.synchronize()
    return 1 + len(trainer.side), [(sl.params.clone(), sl.grads.clone()) for sl in slots]


STREAM_CASES = [
    ("wl2-4layers-f32-dropout", 2, 4, 128, False),
    ("wl4-1layer-T256-bf16-groups", 4, 1, 256, False),
    ("wl5-3layers-T256-dora-stacked-slots", 5, 3, 256, True),
]


@pytest.mark.parametrize("name,wl,layers,tokens,together", STREAM_CASES,
                         ids=[c[0] for c in STREAM_CASES])
def test_streams_give_bitwise_the_one_stream_results(name, wl, layers, tokens, together):
    """Layer groups spread over three streams, each with its own workspace,
    keep every linear's call order, so two updates give bitwise the adapters
    and gradients of the one-stream schedule."""
    cfg = WL.get_config(wl)
    _say("streams", name)
    inputs = _stream_inputs(cfg, layers, tokens)
    n1, one = _trained(cfg, inputs, tokens, 2, 1, together)
    n3, three = _trained(cfg, inputs, tokens, 2, 3, together)
    assert n1 == 1 and n3 == 3
    for (p1, g1), (p3, g3) in zip(one, three):
        assert torch.equal(p1, p3)
        assert torch.equal(g1, g3)


def _fresh(cfg, inputs, tokens, together):
    """A new trainer and freshly initialised slots over the seeded inputs."""
    Wq, per_slot = inputs
    model = S.FrozenModel(cfg, Wq)
    trainer = S.Trainer(cfg, model, tokens=tokens, slots=cfg.slots if together else 1)
    slots = []
    for si, (a, b, _) in enumerate(per_slot):
        slot = S.Slot(cfg, model, a, b, cfg.seeds[si])
        if cfg.dora:
            trainer.init_dora(slot)
        slots.append(slot)
    return trainer, slots, [ch for _, _, ch in per_slot]


def _advance(trainer, slots, chunks, steps, together):
    for _ in range(steps):
        sts = (trainer.step_slots(slots, chunks) if together else
               [trainer.step(sl, ch) for sl, ch in zip(slots, chunks)])
        assert not any(st.vetoed for st in sts)


RESUME_CASES = [
    ("wl2-2layers-f32-dropout", 2, 2, 128, False),
    ("wl4-1layer-T256-cosine", 4, 1, 256, False),
    ("wl5-1layer-T256-dora-stacked-slots", 5, 1, 256, True),
]


@pytest.mark.parametrize("name,wl,layers,tokens,together", RESUME_CASES,
                         ids=[c[0] for c in RESUME_CASES])
def test_resume_from_copied_state_is_bitwise(name, wl, layers, tokens, together):
    """A slot's whole state is its caller-owned buffers (A, B and DoRA
    magnitude in the params arena, Adam m and v) plus its counters t and k
    and its seed; the DoRA norms are derived from A and B.  k + j updates in
    one run equal k updates, a copy of that state to the host and into a
    fresh trainer and slots, then j updates: bitwise."""
    cfg = WL.get_config(wl)
    _say("resume", name)
    inputs = _stream_inputs(cfg, layers, tokens)
    k, j = 2, 2
    tr, slots, chunks = _fresh(cfg, inputs, tokens, together)
    _advance(tr, slots, chunks, k + j, together)
    straight = [(sl.params.clone(), sl.m.clone(), sl.v.clone(), sl.t, sl.k) for sl in slots]
    tr, slots, chunks = _fresh(cfg, inputs, tokens, together)
    _advance(tr, slots, chunks, k, together)
    saved = [(sl.params.cpu(), sl.m.cpu(), sl.v.cpu(), sl.t, sl.k) for sl in slots]
    del tr, slots
    tr, slots, chunks = _fresh(cfg, inputs, tokens, together)
    for sl, (p, m, v, t, kk) in zip(slots, saved):
        sl.params.copy_(p)
        sl.m.copy_(m)
        sl.v.copy_(v)
        sl.t, sl.k = t, kk
    if cfg.dora:   # the norms are derived from the restored A and B
        tr.refresh_dora(slots)
    _advance(tr, slots, chunks, j, together)
    torch.cuda.synchronize()
    for sl, (p, m, v, t, kk) in zip(slots, straight):
        assert (sl.t, sl.k) == (t, kk) == (k + j, k + j)
        assert torch.equal(sl.params, p)
        assert torch.equal(sl.m, m)
        assert torch.equal(sl.v, v)


def test_refresh_on_one_stream_equals_spread_refresh():
    """The refresh's per-stream calls are rebuilt when the trainer's side
    streams are set aside (the bench's one-stream pass); the norms are the
    same bits either way, and both slots' norms match the oracle."""
    cfg = WL.get_config(5)
    inputs = _stream_inputs(cfg, 2, 256)
    tr, slots, _ = _fresh(cfg, inputs, 256, True)
    assert tr.side, "the DoRA workload spreads two layers over two streams"
    tr.refresh_dora(slots)
    spread = [{k: v.clone() for k, v in sl.norm.items()} for sl in slots]
    side, side_ws = tr.side, tr.side_ws
    tr.side, tr.side_ws = [], []
    for sl in slots:
        for v in sl.norm.values():
            v.fill_(float("nan"))
    tr.refresh_dora(slots)
    tr.side, tr.side_ws = side, side_ws
    s = O.scaling(cfg.alpha, cfg.rank, cfg.scaling)
    for sl, ref in zip(slots, spread):
        for key, v in sl.norm.items():
            assert torch.equal(v, ref[key]), key
            W = np64(tr.model.W[key].float())
            want = O.dora_row_norms(W, np64(sl.A[key]), np64(sl.B[key]), s)
            assert rel_err(v, want) <= 1e-5, key


def test_streams_capped_by_layer_groups():
    cfg = WL.get_config(1)
    W = WL.linear_inputs(cfg, 0, cfg.projections[0], chunks=0)["W"].to(DEV)
    trainer = S.Trainer(cfg, S.FrozenModel(cfg, {(0, cfg.projections[0].ordinal): W}), streams=4)
    assert trainer.side == []


def test_group_call_matches_the_group_entry_points():
    """GroupCall marshals the fixed arguments once and reuses X and dY
    pointers while the tensors stay the same; over calls that switch X and
    dY (and use dropout) it gives bitwise the results of lora_forward_group
    and lora_backward_group."""
    T, K, r, Ns = 128, 256, 8, (256, 64)
    cases = [_gpu(_linear_case(T, K, N, r, seed=30 + i)) for i, N in enumerate(Ns)]
    Xs = [WL.draw((T, K), (931, i, 0, 0, 0, "X"), "normal", 1.0, DEV) for i in range(2)]
    dYs = [[WL.draw((T, N), (932, i, j, 0, 0, "dY"), "normal", 1.0, DEV) for j, N in enumerate(Ns)]
           for i in range(2)]
    lins = [L.make_linear(c["Wq"], c["A"], c["B"], 2.0, T) for c in cases]
    order = [0, 1, 1, 0]

    def outputs():
        return dict(Y=[torch.empty(T, N, device=DEV) for N in Ns],
                    U=[torch.empty(T, r, device=DEV) for _ in Ns],
                    dX=[torch.empty(T, K, device=DEV) for _ in Ns],
                    dA=[torch.empty(r, K, device=DEV) for _ in Ns],
                    dB=[torch.empty(N, r, device=DEV) for N in Ns])

    def drops(step):
        return [L.make_dropout(5, step, 0, 0, j, 0.1) for j in range(len(Ns))]

    ws = torch.empty(L.lora_group_workspace_bytes(lins), dtype=torch.uint8, device=DEV)
    a, b = outputs(), outputs()
    ra, rb = [], []
    call = L.GroupCall(lins, b["Y"], b["U"], None, b["dX"], b["dA"], b["dB"], None, ws)
    for step, i in enumerate(order):
        L.lora_forward_group(lins, Xs[i], a["Y"], a["U"], None, drops(step), ws)
        L.lora_backward_group(lins, Xs[i], dYs[i], a["U"], None, a["dX"], a["dA"], a["dB"],
                              accumulate=step > 0, drops=drops(step), ws=ws)
        ra.append([t.clone() for n in ("Y", "U", "dX") for t in a[n]])
        d = call.dropouts(drops(step))
        call.forward(Xs[i], d)
        call.backward(Xs[i], dYs[i], accumulate=step > 0, drops=d)
        rb.append([t.clone() for n in ("Y", "U", "dX") for t in b[n]])
    torch.cuda.synchronize()
    for x, y in zip(ra, rb):
        for u, v in zip(x, y):
            assert torch.equal(u, v)
    for n in ("dA", "dB"):
        for u, v in zip(a[n], b[n]):
            assert torch.equal(u, v)
    assert not torch.equal(ra[0][0], ra[1][0])   # the switched inputs did change Y


def test_invalid_arguments_raise_before_work():
    T, K, N, r = 128, 2048, 2048, 8          # a shape that needs split partials
    c = _gpu(_linear_case(T, K, N, r))
    lin = L.make_linear(c["Wq"], c["A"], c["B"], 2.0, T)
    assert L.lora_workspace_bytes(lin) > 1024
    Y = torch.zeros(T, N, device=DEV)
    U = torch.zeros(T, r, device=DEV)
    with pytest.raises(L.LoraError) as e:
        L.lora_forward(lin, c["X"], Y, U, None, None, torch.empty(16, device=DEV, dtype=torch.uint8))
    assert e.value.status == -5
    bad = L.make_dropout(1, 0, 0, 0, 0, 1.5)
    with pytest.raises(L.LoraError) as e:
        L.lora_forward(lin, c["X"], Y, U, None, bad, None)
    assert e.value.status == -1
    assert torch.count_nonzero(Y).item() == 0 and torch.count_nonzero(U).item() == 0


def test_undersized_buffers_are_refused_on_the_host():
    """A tensor smaller than the descriptor says raises before any launch,
    in the single, group and slot calls alike."""
    T, K, N, r = 64, 136, 264, 8
    c = _gpu(_linear_case(T, K, N, r, seed=5))
    lin = L.make_linear(c["Wq"], c["A"], c["B"], 2.0, T)
    Y = torch.zeros(T, N, device=DEV)
    U = torch.zeros(T, r, device=DEV)
    ws = torch.empty(max(256, L.lora_workspace_bytes(lin)), device=DEV, dtype=torch.uint8)
    with pytest.raises(ValueError, match="Y holds"):
        L.lora_forward(lin, c["X"], Y[: T - 1], U, None, None, ws)
    with pytest.raises(ValueError, match=r"dY\[1\] holds"):
        L.lora_backward_group([lin, lin], c["X"], [c["dY"], c["dY"][:, :8].contiguous()], [U, U],
                              None, None, [torch.zeros(r, K, device=DEV)] * 2,
                              [torch.zeros(N, r, device=DEV)] * 2, ws=ws)
    with pytest.raises(ValueError, match=r"X\[0\] holds"):
        L.lora_forward_slots([lin, lin], [c["X"][:1], c["X"]], [Y, Y], [U, U], None, None, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(Y).item() == 0 and torch.count_nonzero(U).item() == 0


@pytest.mark.parametrize("T,K,N,r", [(128, 2048, 2048, 8), (300, 520, 1096, 16)])
def test_workspace_contents_do_not_matter(T, K, N, r):
    """The workspace only carries split partials that each call writes before
    reading: a garbage-filled workspace gives bitwise the results of a zeroed
    one, and repeated calls on one workspace stay equal."""
    c = _gpu(_linear_case(T, K, N, r, seed=12))
    lin = L.make_linear(c["Wq"], c["A"], c["B"], 2.0, T)
    nb = L.lora_workspace_bytes(lin)
    outs = []
    for fill in ("zero", "garbage", "reuse"):
        if fill != "reuse":
            ws = torch.zeros(nb, device=DEV, dtype=torch.uint8)
            if fill == "garbage":
                ws.random_(0, 256)
        drop = L.make_dropout(7, 1, 0, 0, 2, 0.1)
        Y = torch.empty(T, N, device=DEV)
        U = torch.empty(T, r, device=DEV)
        dX = torch.empty(T, K, device=DEV)
        dA = torch.empty(r, K, device=DEV)
        dB = torch.empty(N, r, device=DEV)
        L.lora_forward(lin, c["X"], Y, U, None, drop, ws)
        L.lora_backward(lin, c["X"], c["dY"], U, None, dX, dA, dB, None, False, drop, ws)
        torch.cuda.synchronize()
        outs.append((Y, U, dX, dA, dB))
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)


# ------------------------------------------------------------- groups -------
def _group_case(T, K, Ns, rs, seed, fmts=None):
    """Linears that read one X: per-linear W (float32, or the given formats),
    A, B, dY; one shared X."""
    fmts = fmts or ["f32"] * len(Ns)
    cs = [_linear_case(T, K, N, r, f, seed=seed + i)
          for i, (N, r, f) in enumerate(zip(Ns, rs, fmts))]
    for c in cs[1:]:
        c["X"] = cs[0]["X"]
    return cs


def _run_linears(cs, s, p, grouped, steps=2):
    """Forward + backward of every linear over `steps` chunks (accumulating),
    through the group calls or one linear at a time."""
    gs = [_gpu(c) for c in cs]
    T, K = gs[0]["X"].shape
    lins = [L.make_linear(g["Wq"], g["A"], g["B"], s, T) for g in gs]
    nanf = float("nan")
    out = {n: [] for n in ("Y", "U", "dX", "dA", "dB")}
    for g, lin in zip(gs, lins):
        N, r = g["W"].shape[0], g["A"].shape[0]
        out["Y"].append(torch.full((T, N), nanf, device=DEV))
        out["U"].append(torch.full((T, r), nanf, device=DEV))
        out["dX"].append(torch.full((T, K), nanf, device=DEV))
        out["dA"].append(torch.full((r, K), nanf, device=DEV))
        out["dB"].append(torch.full((N, r), nanf, device=DEV))
    if grouped:
        ws = torch.empty(max(256, L.lora_group_workspace_bytes(lins)), device=DEV, dtype=torch.uint8)
    else:
        ws = torch.empty(max(256, max(L.lora_workspace_bytes(l) for l in lins)), device=DEV,
                         dtype=torch.uint8)
    for step in range(steps):
        drops = [L.make_dropout(1234, 3, step, 5, i, p) if p > 0 else None for i in range(len(gs))]
        X = gs[0]["X"] if step == 0 else gs[0]["X"] * 0.5
        dYs = [g["dY"] if step == 0 else g["dY"] * -1.5 for g in gs]
        if grouped:
            L.lora_forward_group(lins, X, out["Y"], out["U"], None, drops, ws)
            L.lora_backward_group(lins, X, dYs, out["U"], None, out["dX"], out["dA"], out["dB"],
                                  None, accumulate=step > 0, drops=drops, ws=ws)
        else:
            for i, lin in enumerate(lins):
                L.lora_forward(lin, X, out["Y"][i], out["U"][i], None, drops[i], ws)
                L.lora_backward(lin, X, dYs[i], out["U"][i], None, out["dX"][i], out["dA"][i],
                                out["dB"][i], None, accumulate=step > 0, drop=drops[i], ws=ws)
    torch.cuda.synchronize()
    return out


GROUP_CASES = [
    # name, T, K, [N per linear], [r per linear], dropout p
    ("tinyllama-wq-wv", 128, 2048, [2048, 256], [8, 8], 0.05),
    ("ragged-pair", 100, 1000, [600, 264], [8, 12], 0.1),
    ("mixed-rank-pair", 128, 1024, [512, 768], [8, 40], 0.1),     # one linear off the split path
    ("triple", 72, 520, [264, 136, 520], [4, 8, 16], 0.1),          # more than two: one at a time
    ("bf16-pair", 64, 264, [136, 272], [8, 8], 0.1),
    ("q4_k-q6_k-pair", 96, 512, [264, 136], [8, 16], 0.1),        # a quantized base mixes formats
]


@pytest.mark.parametrize("case", GROUP_CASES, ids=[c[0] for c in GROUP_CASES])
def test_group_calls_equal_single_calls(case):
    """The group calls give bitwise the results of calling each linear alone
    (the same kernels and fixed-order sums, only sharing launches)."""
    name, T, K, Ns, rs, p = case
    _say("group", name)
    fmts = ["q4_k", "q6_k"] if name.startswith("q4_k-q6_k") else None
    cs = _group_case(T, K, Ns, rs, seed=zlib.crc32(name.encode()) % 1000, fmts=fmts)
    if name.startswith("bf16"):
        for c in cs:
            c["Wq"] = c["W"].to(torch.bfloat16)
            c["W"] = c["Wq"].float()
    a = _run_linears(cs, 2.0, p, grouped=True)
    b = _run_linears(cs, 2.0, p, grouped=False)
    for n in a:
        for i in range(len(cs)):
            assert torch.isfinite(a[n][i]).all(), (n, i)
            assert torch.equal(a[n][i], b[n][i]), (n, i)


def test_group_matches_oracle():
    """One chunk of the TinyLlama-shaped wq+wv group against the oracle."""
    cs = _group_case(128, 2048, [2048, 256], [8, 8], seed=41)
    gs = [_gpu(c) for c in cs]
    lins = [L.make_linear(g["Wq"], g["A"], g["B"], 2.0, 128) for g in gs]
    ws = torch.empty(L.lora_group_workspace_bytes(lins), device=DEV, dtype=torch.uint8)
    dk = [(1234, 1, 0, 7, 0), (1234, 1, 0, 7, 2)]
    drops = [L.make_dropout(*k, 0.05) for k in dk]
    Y = [torch.empty(128, g["W"].shape[0], device=DEV) for g in gs]
    U = [torch.empty(128, 8, device=DEV) for g in gs]
    dX = [torch.empty(128, 2048, device=DEV) for g in gs]
    dA = [torch.empty(8, 2048, device=DEV) for g in gs]
    dB = [torch.empty(g["W"].shape[0], 8, device=DEV) for g in gs]
    L.lora_forward_group(lins, gs[0]["X"], Y, U, None, drops, ws)
    L.lora_backward_group(lins, gs[0]["X"], [g["dY"] for g in gs], U, None, dX, dA, dB, None,
                          drops=drops, ws=ws)
    torch.cuda.synchronize()
    for i, c in enumerate(cs):
        ref = _oracle(c, 2.0, 0.05, dk[i])
        got = dict(Y=Y[i], U=U[i], dX=dX[i], dA=dA[i], dB=dB[i])
        for n, t in got.items():
            e = rel_err(t, ref[n])
            _say(f"  linear {i} {n}: rel err {e:.3e}")
            assert e <= 1e-4, (i, n, e)


def test_group_rejects_mismatched_linears():
    cs = [_gpu(_linear_case(64, 128, 64, 4, seed=1)), _gpu(_linear_case(64, 256, 64, 4, seed=2))]
    lins = [L.make_linear(c["Wq"], c["A"], c["B"], 1.0, 64) for c in cs]
    Y = [torch.zeros(64, 64, device=DEV) for _ in cs]
    U = [torch.zeros(64, 4, device=DEV) for _ in cs]
    ws = torch.empty(1 << 20, device=DEV, dtype=torch.uint8)
    with pytest.raises(L.LoraError) as e:
        L.lora_forward_group(lins, cs[0]["X"], Y, U, None, None, ws)
    assert e.value.status == -2
    assert all(torch.count_nonzero(y).item() == 0 for y in Y)


# ---------------------------------------------------------- merge -----------
MERGE_CASES = [
    # W dtype, N, K, r, DoRA
    ("f32", 100, 84, 8, False),       # ragged rows, partial last chunk
    ("bf16", 45, 100, 12, True),      # rows not 16-byte aligned: element loads and stores
    ("bf16", 264, 136, 64, False),
    ("f32", 33, 4097, 128, True),     # rank 128, odd K
    ("bf16", 2560, 9728, 64, True),   # DoRA workload shapes (wdown, wup)
    ("bf16", 9728, 2560, 32, False),
    ("q4_k", 264, 512, 32, True),     # merge of an adapter into a quantized base
    ("q6_k", 136, 768, 16, False),
    ("q8_0", 45, 544, 8, True),
]


@pytest.mark.parametrize("wd_,N,K,r,dora", MERGE_CASES,
                         ids=[f"{c[0]}-{c[1]}x{c[2]}-r{c[3]}{'-dora' if c[4] else ''}" for c in MERGE_CASES])
def test_merge_parity(wd_, N, K, r, dora):
    c = _linear_case(8, K, N, r, wd_, seed=13, b_std=0.05)
    g = _gpu(c)
    s = 1.3
    mag = nrm = None
    if dora:
        mag = torch.rand(N, device=DEV) + 0.5
        nrm = torch.empty(N, device=DEV)
        L.lora_dora_row_norms(L.make_linear(g["Wq"], g["A"], g["B"], s, 8), nrm)
    lin = L.make_linear(g["Wq"], g["A"], g["B"], s, 8, mag, nrm)
    W, A, B = np64(c["W"]), np64(c["A"]), np64(c["B"])
    m64 = np64(mag) if dora else None
    n64 = O.dora_row_norms(W, A, B, s) if dora else None
    if dora:
        assert rel_err(nrm, n64) <= 1e-5
    # float32 output
    out = torch.full((N, K), float("nan"), device=DEV)
    rm = torch.full((1,), float("nan"), device=DEV, dtype=torch.float64)
    L.lora_merge(lin, out, rm)
    ref, _ = O.merge(W, A, B, s, m64, n64, "f32")
    assert rel_err(out, ref) <= 1e-5
    assert rm.item() == 0.0
    # bfloat16 output: each element within one bf16 step of the oracle's
    # rounding (the float32 sums may sit on the other side of a tie), plus
    # the float32 sum's own error, about 2e-6 of the matrix scale (it shows
    # where W and s B A nearly cancel); the RMSE of the rounding close to the
    # oracle's
    outb = torch.full((N, K), float("nan"), device=DEV, dtype=torch.bfloat16)
    L.lora_merge(lin, outb, rm)
    refb, rmse = O.merge(W, A, B, s, m64, n64, "bf16")
    got = np64(outb.float())
    step = np.abs(refb) * 2.0**-7 + 2e-6 * np.abs(ref).max()
    assert np.all(np.abs(got - refb) <= step)
    assert (got != refb).mean() < 1e-3
    assert abs(rm.item() - rmse) <= 1e-3 * rmse


def test_merge_of_zero_adapter_is_exact():
    c = _linear_case(8, 2560, 1024, 32, "bf16", seed=14)
    g = _gpu(c)
    B0 = torch.zeros_like(g["B"])   # held: the descriptor keeps only its address
    lin = L.make_linear(g["Wq"], g["A"], B0, 2.0, 8)
    outb = torch.empty_like(g["Wq"])
    rm = torch.full((1,), float("nan"), device=DEV, dtype=torch.float64)
    L.lora_merge(lin, outb, rm)
    assert torch.equal(outb, g["Wq"]) and rm.item() == 0.0


def test_merge_checks_its_workspace():
    c = _linear_case(8, 512, 64, 8, "bf16", seed=15)
    g = _gpu(c)
    lin = L.make_linear(g["Wq"], g["A"], g["B"], 1.0, 8)
    need = L.lora_merge_workspace_bytes(lin)
    outb = torch.empty_like(g["Wq"])
    rm = torch.zeros(1, device=DEV, dtype=torch.float64)
    with pytest.raises(L.LoraError):
        L.lora_merge(lin, outb, rm, torch.empty(need - 8, device=DEV, dtype=torch.uint8))


# ------------------------------------------------------------ slots ---------
def _slot_cases(T, K, N, r, n, seed, w_dtype="bf16"):
    """n adapter slots over one bf16 (or quantized) W: own X, dY, A, B per slot."""
    cs = [_linear_case(T, K, N, r, w_dtype, seed=seed + i, b_std=0.05) for i in range(n)]
    for c in cs[1:]:
        c["Wq"], c["W"] = cs[0]["Wq"], cs[0]["W"]
    return cs


def _run_slots(cs, s, p, together, dora=False, steps=2):
    """Forward + backward of every slot over `steps` chunks (accumulating),
    through the slot calls or one slot at a time."""
    gs = [_gpu(c) for c in cs]
    for g in gs[1:]:                # the slots share one device copy of W
        g["Wq"], g["W"] = gs[0]["Wq"], gs[0]["W"]
    T, K = gs[0]["X"].shape
    N, r = gs[0]["W"].shape[0], gs[0]["A"].shape[0]
    mags, nrms = [None] * len(gs), [None] * len(gs)
    if dora:
        for i, g in enumerate(gs):
            mags[i] = torch.rand(N, device=DEV) + 0.5
            nrms[i] = torch.empty(N, device=DEV)
            L.lora_dora_row_norms(L.make_linear(g["Wq"], g["A"], g["B"], s, T), nrms[i])
    lins = [L.make_linear(g["Wq"], g["A"], g["B"], s, T, mags[i], nrms[i]) for i, g in enumerate(gs)]
    nanf = float("nan")
    names = ("Y", "U", "dX", "dA", "dB") + (("Z", "dm") if dora else ())
    shapes = dict(Y=(T, N), U=(T, r), dX=(T, K), dA=(r, K), dB=(N, r), Z=(T, N), dm=(N,))
    out = {n: [torch.full(shapes[n], nanf, device=DEV) for _ in gs] for n in names}
    ws = torch.empty(max(L.lora_slots_workspace_bytes(lins),
                         max(L.lora_workspace_bytes(l) for l in lins)), device=DEV, dtype=torch.uint8)
    for step in range(steps):
        drops = [L.make_dropout(1234 + i, 3, step, 5, 4, p) if p > 0 else None for i in range(len(gs))]
        X = [g["X"] if step == 0 else g["X"] * 0.5 for g in gs]
        dYs = [g["dY"] if step == 0 else g["dY"] * -1.5 for g in gs]
        Z = out["Z"] if dora else None
        dm = out["dm"] if dora else None
        if together:
            L.lora_forward_slots(lins, X, out["Y"], out["U"], Z, drops, ws)
            L.lora_backward_slots(lins, X, dYs, out["U"], Z, out["dX"], out["dA"], out["dB"], dm,
                                  accumulate=step > 0, drops=drops, ws=ws)
        else:
            for i, lin in enumerate(lins):
                L.lora_forward(lin, X[i], out["Y"][i], out["U"][i], Z[i] if dora else None,
                               drops[i], ws)
                L.lora_backward(lin, X[i], dYs[i], out["U"][i], Z[i] if dora else None,
                                out["dX"][i], out["dA"][i], out["dB"][i], dm[i] if dora else None,
                                accumulate=step > 0, drop=drops[i], ws=ws)
    torch.cuda.synchronize()
    return out, mags, nrms


SLOT_CASES = [
    # name, T, K, N, r, slots, dropout, DoRA
    ("pair-stacked", 256, 264, 520, 16, 2, 0.1, False),
    ("pair-stacked-dora", 256, 520, 264, 32, 2, 0.1, True),
    ("four-stacked", 256, 136, 272, 8, 4, 0.0, False),
    ("qwen-wgate-pair", 512, 2560, 9728, 64, 2, 0.1, True),
    ("q4_k-pair-stacked", 256, 512, 264, 16, 2, 0.1, False, "q4_k"),
]


@pytest.mark.parametrize("case", SLOT_CASES, ids=[c[0] for c in SLOT_CASES])
def test_slots_match_oracle(case):
    """Each slot of a stacked slot call against the oracle (two accumulated
    chunks), at the bf16-W bar."""
    name, T, K, N, r, n, p, dora = case[:8]
    wd = case[8] if len(case) > 8 else "bf16"
    _say("slots", name)
    cs = _slot_cases(T, K, N, r, n, seed=zlib.crc32(name.encode()) % 1000, w_dtype=wd)
    got, mags, nrms = _run_slots(cs, 1.5, p, together=True, dora=dora)
    for i, c in enumerate(cs):
        refs = []
        for step in range(2):
            ci = dict(c)
            if step:
                ci["X"], ci["dY"] = c["X"] * 0.5, c["dY"] * -1.5
            m = np64(mags[i]) if dora else None
            nr = O.dora_row_norms(np64(c["W"]), np64(c["A"]), np64(c["B"]), 1.5) if dora else None
            if dora:
                assert rel_err(nrms[i], nr) <= 1e-5
            refs.append(_oracle(ci, 1.5, p, (1234 + i, 3, step, 5, 4), m, nr))
        last = refs[-1]
        checks = dict(Y=last["Y"], U=last["U"], dX=last["dX"], dA=refs[0]["dA"] + last["dA"],
                      dB=refs[0]["dB"] + last["dB"])
        if dora:
            checks["Z"] = last["Z"]
            checks["dm"] = refs[0]["dmag"] + last["dmag"]
        for nme, ref in checks.items():
            e = rel_err(got[nme][i], ref)
            _say(f"  slot {i} {nme}: rel err {e:.3e}")
            assert e <= 2e-2 if nme in ("Y", "dX", "Z", "dm") else e <= 1e-4, (i, nme, e)


def test_direct_operand_stacked_slots_match_oracle(bf16_config_5):
    """Two stacked slots on the direct-operand loop: the slots' bf16 copies
    of X and g are fragment-tiled one above another (forward 1024 whole
    columns; dX 640 columns, the last tile ragged)."""
    test_slots_match_oracle(("direct-pair-stacked-dora", 256, 640, 1024, 32, 2, 0.1, True))


FROM_Y_CASES = [
    # name, T, K, N, r, w dtype, dropout
    ("bf16-direct", 256, 640, 1024, 32, "bf16", 0.1),
    ("bf16-ragged", 96, 600, 1000, 16, "bf16", 0.1),
    ("f32-ragged", 100, 264, 136, 8, "f32", 0.0),
]


@pytest.mark.parametrize("case", FROM_Y_CASES, ids=[c[0] for c in FROM_Y_CASES])
def test_dora_backward_from_y(case):
    """dora_from_y: the forward writes no Z and the backward takes the
    forward's Y in its place (dm = sum_t dY Y / mag).  Every output matches
    the oracle, and dm matches the Z-mode call to float32 rounding."""
    name, T, K, N, r, wd_, p = case
    _say("dora from y", name)
    c = _linear_case(T, K, N, r, wd_, seed=zlib.crc32(name.encode()) % 1000, dy_std=1e-2, b_std=0.05)
    s, dk = 2.0, (99, 1, 2, 3, 4)
    z = _run_gpu(c, s, p, dk, True)            # Z mode: mag, norm, and the reference run
    g = z["g"]
    lin = L.make_linear(g["Wq"], g["A"], g["B"], s, T, z["mag"], z["norm"], dora_from_y=True)
    ws = torch.empty(L.lora_workspace_bytes(lin), device=DEV, dtype=torch.uint8)
    drop = L.make_dropout(*dk, p) if p > 0 else None
    nanf = float("nan")
    Y, U = torch.full((T, N), nanf, device=DEV), torch.full((T, r), nanf, device=DEV)
    L.lora_forward(lin, g["X"], Y, U, None, drop, ws)
    dX, dA = torch.full((T, K), nanf, device=DEV), torch.full((r, K), nanf, device=DEV)
    dB, dm = torch.full((N, r), nanf, device=DEV), torch.full((N,), nanf, device=DEV)
    L.lora_backward(lin, g["X"], g["dY"], U, Y, dX, dA, dB, dm, False, drop, ws)
    torch.cuda.synchronize()
    got = dict(Y=Y, U=U, dX=dX, dA=dA, dB=dB, dmag=dm)
    mag, nrm = _dora_vectors(z, c, s)
    ref = _oracle(c, s, p, dk, mag, nrm)
    for n in got:
        assert torch.isfinite(got[n]).all(), n
        e = rel_err(got[n], ref[n])
        _say(f"  {n}: rel err {e:.3e}")
        assert e <= TOL[wd_], (n, e)
    assert rel_err(dm, z["dmag"]) <= 1e-5


def test_dora_backward_from_y_stacked_slots():
    """The same through the stacked slot calls (each slot's own mag)."""
    cs = _slot_cases(256, 640, 1024, 32, 2, seed=91)
    gs = [_gpu(c) for c in cs]
    for g in gs[1:]:
        g["Wq"], g["W"] = gs[0]["Wq"], gs[0]["W"]
    T, K, N, r = 256, 640, 1024, 32
    mags = [torch.rand(N, device=DEV) + 0.5 for _ in gs]
    nrms = [torch.empty(N, device=DEV) for _ in gs]
    for g, nr in zip(gs, nrms):
        L.lora_dora_row_norms(L.make_linear(g["Wq"], g["A"], g["B"], 2.0, T), nr)
    out = {}
    for from_y in (False, True):
        lins = [L.make_linear(g["Wq"], g["A"], g["B"], 2.0, T, m, nr, dora_from_y=from_y)
                for g, m, nr in zip(gs, mags, nrms)]
        ws = torch.empty(L.lora_slots_workspace_bytes(lins), device=DEV, dtype=torch.uint8)
        drops = [L.make_dropout(5 + i, 1, 0, 2, 3, 0.1) for i in range(2)]
        Y = [torch.empty(T, N, device=DEV) for _ in gs]
        U = [torch.empty(T, r, device=DEV) for _ in gs]
        Z = None if from_y else [torch.empty(T, N, device=DEV) for _ in gs]
        L.lora_forward_slots(lins, [g["X"] for g in gs], Y, U, Z, drops, ws)
        dX = [torch.empty(T, K, device=DEV) for _ in gs]
        dA = [torch.empty(r, K, device=DEV) for _ in gs]
        dB = [torch.empty(N, r, device=DEV) for _ in gs]
        dm = [torch.empty(N, device=DEV) for _ in gs]
        L.lora_backward_slots(lins, [g["X"] for g in gs], [g["dY"] for g in gs], U, Y if from_y else Z,
                              dX, dA, dB, dm, accumulate=False, drops=drops, ws=ws)
        torch.cuda.synchronize()
        out[from_y] = dict(Y=Y, dX=dX, dA=dA, dB=dB, dm=dm)
    for n in ("Y", "dX", "dA", "dB"):
        for i in range(2):
            assert torch.equal(out[True][n][i], out[False][n][i]), (n, i)
    for i in range(2):
        assert rel_err(out[True]["dm"][i], out[False]["dm"][i]) <= 1e-5, i


def test_dora_from_y_needs_dora():
    c = _gpu(_linear_case(64, 64, 64, 4, "f32", seed=3))
    lin = L.make_linear(c["Wq"], c["A"], c["B"], 1.0, 64, dora_from_y=True)
    ws = torch.empty(max(L.lora_workspace_bytes(lin), 256), device=DEV, dtype=torch.uint8)
    Y, U = torch.zeros(64, 64, device=DEV), torch.zeros(64, 4, device=DEV)
    with pytest.raises(L.LoraError) as e:
        L.lora_forward(lin, c["X"], Y, U, None, None, ws)
    assert e.value.status == -1   # LORA_E_INVALID


def _pinned(cfg, fn):
    L.lora_set_bf16_config(cfg)
    try:
        return fn()
    finally:
        L.lora_set_bf16_config(-1)


MASK_BIT_CASES = [
    # name, T, K, N, r (the dX product: K output columns, contraction N)
    ("ragged-cols", 96, 600, 1088, 16),       # last keep word partial; waves past the columns
    ("ragged-rows", 288, 1000, 640, 32),      # a tile row past the last token
    ("split-contraction", 256, 2560, 512, 64),
    ("rank-128", 128, 640, 1088, 128),        # the mask applied to each of two rank chunks
]


@pytest.mark.parametrize("case", MASK_BIT_CASES, ids=[c[0] for c in MASK_BIT_CASES])
def test_direct_dx_stored_keep_bits_match_hashed_mask(case):
    """dX on the direct-operand loop applies the LoRA term's dropout mask
    from the keep bits that k4 stores; configuration 1 hashes the mask
    itself.  The two agree up to the frozen product's summation order: one
    wrong bit would move an element by a whole LoRA term, far above 1e-5."""
    name, T, K, N, r = case
    _say("keep bits", name)
    c = _linear_case(T, K, N, r, "bf16", seed=zlib.crc32(name.encode()) % 1000, dy_std=1e-2, b_std=0.05)
    dk = (77, 5, 2, 1, 3)
    a = _pinned(1, lambda: _run_gpu(c, 2.0, 0.3, dk, False))
    b = _pinned(5, lambda: _run_gpu(c, 2.0, 0.3, dk, False))
    for n in ("dX", "dA", "dB"):
        assert torch.isfinite(b[n]).all(), n
        e = rel_err(b[n], a[n])
        _say(f"  {n}: rel diff {e:.2e}")
        assert e <= 1e-5, (n, e)


def test_direct_dx_stored_keep_bits_match_hashed_mask_stacked():
    """The same for two stacked slots (each slot's bits, own dropout keys)."""
    cs = _slot_cases(256, 640, 1024, 32, 2, seed=83)
    a, _, _ = _pinned(1, lambda: _run_slots(cs, 2.0, 0.3, together=True))
    b, _, _ = _pinned(5, lambda: _run_slots(cs, 2.0, 0.3, together=True))
    for i in range(2):
        assert torch.isfinite(b["dX"][i]).all(), i
        assert rel_err(b["dX"][i], a["dX"][i]) <= 1e-5, i


@pytest.mark.parametrize("T", [256, 100])
def test_slots_equal_separate_calls(T):
    """Stacked (T a multiple of 256) slot calls agree with separate calls up
    to the frozen products' summation order; unstacked ones (ragged T) are
    the separate calls, bitwise."""
    cs = _slot_cases(T, 264, 136, 8, 2, seed=61)
    a, _, _ = _run_slots(cs, 2.0, 0.1, together=True)
    b, _, _ = _run_slots(cs, 2.0, 0.1, together=False)
    for nme in a:
        for i in range(2):
            assert torch.isfinite(a[nme][i]).all(), (nme, i)
            if T % 256:
                assert torch.equal(a[nme][i], b[nme][i]), (nme, i)
            else:
                assert rel_err(a[nme][i], b[nme][i]) <= 1e-5, (nme, i)


def test_slots_reject_different_w():
    cs = [_gpu(c) for c in _slot_cases(256, 136, 64, 4, 2, seed=71)]
    other = (cs[1]["Wq"].float() * 2).to(torch.bfloat16)
    lins = [L.make_linear(cs[0]["Wq"], cs[0]["A"], cs[0]["B"], 1.0, 256),
            L.make_linear(other, cs[1]["A"], cs[1]["B"], 1.0, 256)]
    Y = [torch.zeros(256, 64, device=DEV) for _ in cs]
    U = [torch.zeros(256, 4, device=DEV) for _ in cs]
    ws = torch.empty(1 << 22, device=DEV, dtype=torch.uint8)
    with pytest.raises(L.LoraError) as e:
        L.lora_forward_slots(lins, [c["X"] for c in cs], Y, U, None, None, ws)
    assert e.value.status == -2
    assert all(torch.count_nonzero(y).item() == 0 for y in Y)
