"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names the fact it checks: published reference values, closed forms,
invariants, a library routine (torch.autograd, torch.optim.AdamW,
numpy.linalg.norm) or brute force on tiny inputs.  CPU only.
"""

import hashlib
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(20261202)


def _rand(*shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- hash ----
def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [int(l) for l in f if l.strip() and not l.startswith("#")]


def test_splitmix64_reference_outputs():
    """SplitMix64 seeded 1234567 reproduces the published first outputs."""
    expect = _golden_ints("splitmix64_seed1234567.txt")
    state, got = 1234567, []
    for _ in expect:
        state, out = O.splitmix64_next(state)
        got.append(out)
    assert got == expect


def test_mix64_array_equals_reference_step():
    """The uint64-array mixer equals the Python-int SplitMix64 output."""
    states = [0, 1, 1234567, 2**63 + 5, 2**64 - 1, 0x0123456789ABCDEF]
    arr = O.mix64(np.array(states, dtype=np.uint64))
    for s, a in zip(states, arr):
        assert int(a) == O.splitmix64_next(s)[1]


def test_dropout_mask_rerun_identical_and_p0_keeps_all():
    a = O.dropout_keep(1234, 3, 1, 5, 2, 64, 96, 0.1)
    b = O.dropout_keep(1234, 3, 1, 5, 2, 64, 96, 0.1)
    assert a.dtype == bool and a.shape == (64, 96)
    assert np.array_equal(a, b)
    assert O.dropout_keep(1234, 3, 1, 5, 2, 16, 16, 0.0).all()


@pytest.mark.parametrize("p", [0.05, 0.1, 0.5])
def test_dropout_keep_fraction_within_5_sigma(p):
    T, K = 512, 512
    keep = O.dropout_keep(7, 0, 0, 0, 0, T, K, p)
    n = T * K
    q = 1.0 - p
    assert abs(keep.mean() - q) < 5.0 * math.sqrt(q * (1 - q) / n)


@pytest.mark.parametrize("which", range(6))
def test_dropout_every_key_changes_the_mask(which):
    """Changing any single key flips about 2p(1-p) of the decisions."""
    p = 0.3
    base = [1234, 2, 1, 7, 2]
    keys = list(base)
    T, K = 256, 256
    ref = O.dropout_keep(*keys, T, K, p)
    if which < 5:
        keys[which] += 1
        other = O.dropout_keep(*keys, T, K, p)
    else:  # token rows: shift by one row
        other = O.dropout_keep(*keys, T + 1, K, p)[1:]
    frac = (ref != other).mean()
    expect = 2 * p * (1 - p)
    assert abs(frac - expect) < 5.0 * math.sqrt(expect * (1 - expect) / (T * K))


def test_dropout_threshold_and_scale_are_the_rounded_definitions():
    assert O.dropout_threshold(0.0) == 0
    assert O.dropout_threshold(0.5) == 1 << 23
    assert O.dropout_threshold(0.05) == 838861      # round(0.05f * 2^24)
    assert O.dropout_scale(0.5) == 2.0
    assert O.dropout_scale(0.1) == float(np.float32(1.0 / 0.9))  # float32 1/(1-p)


# ------------------------------------------------------------- scaling ----
def test_scaling_closed_forms():
    assert O.scaling(8, 4) == 2.0
    assert O.scaling(16, 8) == 2.0
    assert O.scaling(32, 32, "rslora") == pytest.approx(math.sqrt(32), rel=1e-15)
    assert O.scaling(64, 64) == 1.0


# ------------------------------------------------------- forward pins -----
def _lin(T=6, K=7, N=5, r=3, seed=0):
    g = np.random.default_rng(seed)
    return dict(X=g.standard_normal((T, K)), W=g.standard_normal((N, K)) * 0.3,
                A=g.standard_normal((r, K)) * 0.4, B=g.standard_normal((N, r)) * 0.5,
                dY=g.standard_normal((T, N)))


def test_zero_adapter_is_exact_noop():
    """B = 0: Y equals the frozen-only product bitwise and dA is exactly 0."""
    d = _lin(T=32, K=64, N=64, r=4)
    B0 = np.zeros_like(d["B"])
    keep = O.dropout_keep(1, 0, 0, 0, 0, 32, 64, 0.2)
    Y, U, Z = O.forward(d["X"], d["W"], d["A"], B0, 2.0, keep, O.dropout_scale(0.2))
    frozen = np.asarray(d["X"], np.float64) @ np.asarray(d["W"], np.float64).T
    assert np.array_equal(Y, frozen)
    g = O.backward(d["X"], d["dY"], d["W"], d["A"], B0, 2.0, U, keep, O.dropout_scale(0.2))
    assert not g["dA"].any()


def test_zero_adapter_dora_scale_is_exactly_one():
    """DoRA with B = 0 and magnitude = ||W|| rows: c = 1 exactly, so Y = Z."""
    d = _lin(T=8, K=16, N=12, r=2)
    B0 = np.zeros_like(d["B"])
    mag = O.dora_row_norms(d["W"])
    nrm = O.dora_row_norms(d["W"], d["A"], B0, 1.5)
    assert np.array_equal(mag, nrm)
    Y, U, Z = O.forward(d["X"], d["W"], d["A"], B0, 1.5, mag=mag, norm=nrm)
    assert np.array_equal(Y, Z)


def test_merged_weight_forward():
    """X (W + s B A)^T equals the two-branch forward (no dropout)."""
    d = _lin(T=9, K=11, N=13, r=4)
    s = 2.5
    Y, _, _ = O.forward(d["X"], d["W"], d["A"], d["B"], s)
    merged = d["X"] @ (d["W"] + s * d["B"] @ d["A"]).T
    assert np.abs(Y - merged).max() <= 1e-12 * np.abs(merged).max()


def test_rows_norms_match_numpy_linalg():
    d = _lin(T=2, K=19, N=7, r=3)
    ref = np.linalg.norm(d["W"] + 0.7 * d["B"] @ d["A"], axis=1)
    got = O.dora_row_norms(d["W"], d["A"], d["B"], 0.7)
    assert np.allclose(got, ref, rtol=1e-14, atol=0)


# ----------------------------------------------------- backward pins ------
def _loss(X, W, A, B, s, dY, keep, ks, mag=None, nrm=None):
    Y, _, _ = O.forward(X, W, A, B, s, keep, ks, mag, nrm)
    return float((dY * Y).sum())


@pytest.mark.parametrize("dropout,dora", [(0.0, False), (0.3, False), (0.0, True), (0.3, True)])
def test_central_finite_differences(dropout, dora):
    """L = <dY, Y> is linear in each of X, A, B, mag: central differences
    are exact up to rounding, so they pin every gradient."""
    T, K, N, r = 3, 5, 4, 2
    d = _lin(T, K, N, r, seed=3)
    s = 1.7
    keep = O.dropout_keep(9, 1, 0, 2, 3, T, K, dropout) if dropout else None
    ks = O.dropout_scale(dropout) if dropout else 1.0
    mag = np.abs(_rand(N)) + 0.5 if dora else None
    nrm = O.dora_row_norms(d["W"], d["A"], d["B"], s) if dora else None
    X, W, A, B, dY = d["X"], d["W"], d["A"], d["B"], d["dY"]
    _, U, Z = O.forward(X, W, A, B, s, keep, ks, mag, nrm)
    g = O.backward(X, dY, W, A, B, s, U, keep, ks, mag, nrm, Z)
    h = 1e-3
    names = [("X", X, "dX"), ("A", A, "dA"), ("B", B, "dB")]
    if dora:
        names.append(("mag", mag, "dmag"))
    for name, arr, gname in names:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args = dict(X=X, W=W, A=A, B=B, mag=mag)
            plus = arr.copy(); plus[idx] += h
            minus = arr.copy(); minus[idx] -= h
            args[name] = plus
            lp = _loss(args["X"], W, args["A"], args["B"], s, dY, keep, ks, args["mag"], nrm)
            args[name] = minus
            lm = _loss(args["X"], W, args["A"], args["B"], s, dY, keep, ks, args["mag"], nrm)
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(fd - g[gname]).max() <= 1e-9 * max(1.0, np.abs(fd).max()), name


def test_autograd_float64_matches_backward_with_dropout_and_dora():
    """torch.autograd in float64 on the config-1 shapes (plus dropout/DoRA)."""
    T, K, N, r, s, p = 32, 64, 64, 4, 2.0, 0.25
    d = _lin(T, K, N, r, seed=11)
    keep = O.dropout_keep(42, 0, 1, 3, 4, T, K, p)
    ks = O.dropout_scale(p)
    mag = np.abs(_rand(N)) + 0.5
    nrm = O.dora_row_norms(d["W"], d["A"], d["B"], s)
    tX = torch.tensor(d["X"], requires_grad=True)
    tA = torch.tensor(d["A"], requires_grad=True)
    tB = torch.tensor(d["B"], requires_grad=True)
    tm = torch.tensor(mag, requires_grad=True)
    tW = torch.tensor(d["W"])
    tk = torch.tensor(keep, dtype=torch.float64) * ks
    Z = tX @ tW.T + s * ((tX * tk) @ tA.T) @ tB.T
    Y = Z * (tm / torch.tensor(nrm))[None, :]
    Y.backward(torch.tensor(d["dY"]))
    Yo, U, Zo = O.forward(d["X"], d["W"], d["A"], d["B"], s, keep, ks, mag, nrm)
    assert np.abs(Yo - Y.detach().numpy()).max() <= 1e-13 * np.abs(Yo).max()
    g = O.backward(d["X"], d["dY"], d["W"], d["A"], d["B"], s, U, keep, ks, mag, nrm, Zo)
    for ours, ref in ((g["dX"], tX.grad), (g["dA"], tA.grad), (g["dB"], tB.grad), (g["dmag"], tm.grad)):
        ref = ref.numpy()
        assert np.abs(ours - ref).max() <= 1e-12 * np.abs(ref).max()


def test_adjointness_of_frozen_products():
    """<X W^T, V> == <X, V W> (the adjointness test the pages describe)."""
    d = _lin(T=17, K=23, N=19, r=2)
    V = _rand(17, 19)
    Y, _, _ = O.forward(d["X"], d["W"], d["A"], np.zeros_like(d["B"]), 1.0)
    g = O.backward(d["X"], V, d["W"], d["A"], np.zeros_like(d["B"]), 1.0, np.zeros((17, 2)))
    lhs = float((Y * V).sum())
    rhs = float((d["X"] * g["dX"]).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0)


def test_dora_magnitude_gradient_closed_form():
    """B = 0, mag = ||W||: dm_n = sum_t dY[t,n] (X W^T)[t,n] / ||W_n||."""
    d = _lin(T=10, K=12, N=6, r=3)
    B0 = np.zeros_like(d["B"])
    mag = O.dora_row_norms(d["W"])
    nrm = O.dora_row_norms(d["W"], d["A"], B0, 1.0)
    _, U, Z = O.forward(d["X"], d["W"], d["A"], B0, 1.0, mag=mag, norm=nrm)
    g = O.backward(d["X"], d["dY"], d["W"], d["A"], B0, 1.0, U, mag=mag, norm=nrm, Z=Z)
    ref = (d["dY"] * (d["X"] @ d["W"].T)).sum(0) / np.linalg.norm(d["W"], axis=1)
    assert np.allclose(g["dmag"], ref, rtol=1e-13, atol=0)


# -------------------------------------------------------- prepare pins ----
def test_clip_scales_norm_to_exactly_max_norm():
    g = [_rand(40, 7, scale=3.0), _rand(9, scale=5.0)]
    n_pred = 4
    prep = O.grad_prepare(g, n_pred, 1.0)
    assert prep["finite"] and prep["norm"] > 1.0
    scaled = np.sqrt(sum(float(((x * prep["scale"]) ** 2).sum()) for x in g))
    assert scaled == pytest.approx(1.0, rel=1e-6)


def test_unclipped_and_disabled_clip_only_normalise():
    g = [_rand(30, scale=1e-3)]
    prep = O.grad_prepare(g, 128, 1.0)
    assert prep["clip"] == 1.0 and prep["scale"] == float(np.float32(1.0 / 128))
    assert prep["norm"] == pytest.approx(np.linalg.norm(g[0]) / 128, rel=1e-14)
    big = [_rand(30, scale=1e3)]
    prep0 = O.grad_prepare(big, 3, 0.0)
    assert prep0["clip"] == 1.0 and prep0["scale"] == float(np.float32(1.0 / 3))


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_is_vetoed(bad):
    g = [_rand(5), _rand(3)]
    g[1][2] = bad
    assert O.grad_prepare(g, 1, 1.0)["finite"] is False


# ---------------------------------------------------------- AdamW pins ----
def test_first_adamw_step_closed_form():
    """t = 1: delta = -lr_e g'/(|g'| + eps) - [A] lr wd theta."""
    th, g = _rand(50), _rand(50)
    c, lr, wd, ratio, eps = 0.25, 1e-3, 0.1, 4.0, 1e-8
    gp = g * c
    for kind, rate, decay in (("A", lr, wd), ("B", lr * ratio, 0.0), ("mag", lr, 0.0)):
        new, m, v = O.adamw_update(th, g, np.zeros(50), np.zeros(50), kind, lr, 1, c,
                                   weight_decay=wd, plus_ratio=ratio, eps=eps)
        expect = th - rate * gp / (np.abs(gp) + eps) - lr * decay * th
        assert np.allclose(new, expect, rtol=1e-12, atol=1e-15)


def test_adamw_matches_torch_optim_adamw_over_steps():
    """torch.optim.AdamW (float64, two groups: A decayed at lr, B undecayed at
    lr*ratio) equals the oracle over several steps with varying lr."""
    lr, wd, ratio, c = 1e-3, 0.05, 8.0, 0.5
    A0, B0 = _rand(4, 9), _rand(6, 4)
    tA = torch.nn.Parameter(torch.tensor(A0))
    tB = torch.nn.Parameter(torch.tensor(B0))
    opt = torch.optim.AdamW([{"params": [tA], "lr": lr, "weight_decay": wd},
                             {"params": [tB], "lr": lr * ratio, "weight_decay": 0.0}],
                            betas=(0.9, 0.999), eps=1e-8)
    st = {"A": (A0, np.zeros_like(A0), np.zeros_like(A0)),
          "B": (B0, np.zeros_like(B0), np.zeros_like(B0))}
    for t in range(1, 6):
        lr_t = lr * (0.5 + 0.1 * t)
        gA, gB = _rand(4, 9), _rand(6, 4)
        opt.param_groups[0]["lr"] = lr_t
        opt.param_groups[1]["lr"] = lr_t * ratio
        tA.grad = torch.tensor(gA * c)
        tB.grad = torch.tensor(gB * c)
        opt.step()
        for name, gg in (("A", gA), ("B", gB)):
            th, m, v = st[name]
            st[name] = O.adamw_update(th, gg, m, v, name, lr_t, t, c,
                                      weight_decay=wd, plus_ratio=ratio)
    assert np.allclose(st["A"][0], tA.detach().numpy(), rtol=1e-13, atol=1e-16)
    assert np.allclose(st["B"][0], tB.detach().numpy(), rtol=1e-13, atol=1e-16)


# ----------------------------------------------------------- schedule -----
def test_schedule_closed_forms():
    lr, lo, wu, tot = 1e-4, 1e-5, 10, 100
    assert O.lr_at(0, lr, "cosine", wu, tot, lo) == pytest.approx(lr / wu)
    assert O.lr_at(wu - 1, lr, "cosine", wu, tot, lo) == pytest.approx(lr)
    assert O.lr_at(wu, lr, "cosine", wu, tot, lo) == pytest.approx(lr)
    assert O.lr_at((wu + tot) // 2, lr, "cosine", wu, tot, lo) == pytest.approx((lr + lo) / 2)
    assert O.lr_at(tot, lr, "cosine", wu, tot, lo) == pytest.approx(lo)
    assert O.lr_at(tot + 50, lr, "cosine", wu, tot, lo) == pytest.approx(lo)
    assert all(O.lr_at(k, lr) == lr for k in range(20))


# ----------------------------------------------------- whole-step pins ----
def _tiny_setup(T=8, K=12, N=10, r=3, chunks=2, layers=2, dora=False, p=0.0, seed=5):
    g = np.random.default_rng(seed)
    linears, params, norms = {}, {}, {}
    s = 1.5
    for l in range(layers):
        for pj in (0, 2):
            key = (l, pj)
            W = g.standard_normal((N, K)) * 0.2
            linears[key] = W
            params[key] = {"A": g.standard_normal((r, K)) * 0.3, "B": g.standard_normal((N, r)) * 0.1}
            if dora:
                params[key]["mag"] = O.dora_row_norms(W)
                norms[key] = O.dora_row_norms(W, params[key]["A"], params[key]["B"], s)
    chunks_l = []
    for c in range(chunks):
        ch = {}
        for key in linears:
            ch[key] = (g.standard_normal((T, K)), g.standard_normal((T, N)) * 0.1)
        chunks_l.append(ch)
    hp = dict(s=s, p=p, seed=77, n_pred=T * chunks, max_norm=1.0, lr=1e-3,
              weight_decay=0.01, plus_ratio=2.0, dora=dora)
    return O.SlotState(params=params, norms=norms), linears, chunks_l, hp


def test_accumulation_equals_concatenated_chunk():
    """G chunks of T tokens give the update of one chunk of G*T tokens."""
    st1, lin, chunks, hp = _tiny_setup(chunks=3)
    st2 = O.SlotState(params={k: {n: a.copy() for n, a in v.items()} for k, v in st1.params.items()})
    cat = {key: (np.concatenate([c[key][0] for c in chunks]), np.concatenate([c[key][1] for c in chunks]))
           for key in lin}
    O.train_step(st1, lin, chunks, hp)
    O.train_step(st2, lin, [cat], hp)
    for key in lin:
        for n in ("A", "B"):
            assert np.allclose(st1.params[key][n], st2.params[key][n], rtol=1e-12, atol=1e-15)


def _sha(state):
    h = hashlib.sha256()
    for key in sorted(state.params):
        for n in sorted(state.params[key]):
            h.update(np.ascontiguousarray(state.params[key][n]).tobytes())
    return h.hexdigest()


@pytest.mark.parametrize("dora,p", [(False, 0.1), (True, 0.1)])
def test_seeded_runs_give_identical_adapters(dora, p):
    digests = []
    for _ in range(2):
        st, lin, chunks, hp = _tiny_setup(dora=dora, p=p)
        for _ in range(3):
            O.train_step(st, lin, chunks, hp)
        digests.append(_sha(st))
    assert digests[0] == digests[1]


def test_non_finite_gradient_leaves_state_untouched():
    st, lin, chunks, hp = _tiny_setup()
    O.train_step(st, lin, chunks, hp)
    before = _sha(st), st.t, st.k
    moments = {k: {n: a.copy() for n, a in v.items()} for k, v in st.m.items()}
    key = next(iter(lin))
    X, dY = chunks[0][key]
    dY = dY.copy(); dY[0, 0] = np.nan
    chunks[0][key] = (X, dY)
    res = O.train_step(st, lin, chunks, hp)
    assert res["vetoed"]
    assert (_sha(st), st.t, st.k) == before
    for k, v in st.m.items():
        for n, a in v.items():
            assert np.array_equal(a, moments[k][n])


def test_dora_step_refreshes_norms():
    st, lin, chunks, hp = _tiny_setup(dora=True)
    O.train_step(st, lin, chunks, hp)
    for key, W in lin.items():
        pr = st.params[key]
        ref = np.linalg.norm(W + hp["s"] * pr["B"] @ pr["A"], axis=1)
        assert np.allclose(st.norms[key], ref, rtol=1e-14)


# ------------------------------------------------------------ merge ---------
def test_bf16_round_hand_worked_cases():
    # bfloat16 keeps 8 significant bits: near 1 the spacing is 2**-7.
    x = np.array([1.0 + 2.0**-8,          # tie, lower neighbour even -> 1
                  1.0 + 3 * 2.0**-8,      # tie, upper neighbour even -> 1 + 2**-6
                  1.0 + 2.0**-8 + 2.0**-20,   # just above the tie -> up
                  2.0 - 2.0**-9,          # tie at the top of the binade: even is 2.0
                  -(1.0 + 2.0**-8),       # sign is kept
                  0.0, 3.0], dtype=np.float32)
    want = [1.0, 1.0 + 2.0**-6, 1.0 + 2.0**-7, 2.0, -1.0, 0.0, 3.0]
    assert O.bf16_round(x).tolist() == want


def test_merge_with_zero_b_returns_w():
    rng = np.random.default_rng(5)
    W = O.bf16_round(rng.normal(0, 0.02, (12, 20)))      # bf16-representable W
    A = rng.normal(0, 1, (4, 20))
    W_out, rmse = O.merge(W, A, np.zeros((12, 4)), 2.0, out="bf16")
    assert np.array_equal(W_out, W) and rmse == 0.0
    W_out, rmse = O.merge(W, A, np.zeros((12, 4)), 2.0)
    assert np.array_equal(W_out, W) and rmse == 0.0


@pytest.mark.parametrize("dora", [False, True])
def test_merged_weight_reproduces_forward(dora):
    rng = np.random.default_rng(6)
    T, K, N, r, s = 7, 24, 10, 4, 1.5
    X, W = rng.normal(0, 1, (T, K)), rng.normal(0, 0.02, (N, K))
    A, B = rng.normal(0, 0.3, (r, K)), rng.normal(0, 0.1, (N, r))
    mag = nrm = None
    if dora:
        mag = rng.uniform(0.5, 2.0, N)
        nrm = O.dora_row_norms(W, A, B, s)
    Y, _, _ = O.forward(X, W, A, B, s, mag=mag, norm=nrm)
    W_out, _ = O.merge(W, A, B, s, mag, nrm)
    assert np.allclose(X @ W_out.T, Y, rtol=0, atol=1e-6 * np.abs(Y).max())


def test_merge_rmse_of_ties_closed_form():
    # Every merged value is a tie 1 + 2**-8 (rounds to 1) or 1 + 3*2**-8
    # (rounds to 1 + 2**-6): each element is off by exactly 2**-8.
    W = np.where(np.arange(6 * 8).reshape(6, 8) % 2 == 0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8)
    _, rmse = O.merge(W, np.zeros((1, 8)), np.zeros((6, 1)), 1.0, out="bf16")
    assert rmse == 2.0**-8


# ------------------------------------------------ block-quantized frozen W --
from oracle import quant as Q


def _pack_nibbles(codes):
    """Independent packer (pure Python): element 2j -> low nibble of byte j."""
    rows = []
    for row in codes:
        rows.append([int(row[2 * j]) | (int(row[2 * j + 1]) << 4) for j in range(len(row) // 2)])
    return np.array(rows, dtype=np.uint8)


def _pack_crumbs(fields):
    """Independent packer: element 4j+i -> bits 2i..2i+1 of byte j."""
    rows = []
    for row in fields:
        rows.append([sum(int(row[4 * j + i]) << (2 * i) for i in range(4))
                     for j in range(len(row) // 4)])
    return np.array(rows, dtype=np.uint8)


def test_q4_0_decodes_closed_form_codes_per_block_scale():
    # code of element k is k mod 16; block b (32 elements) has d = 2^-(b+3)
    N, K = 2, 96
    codes = np.array([[(k + 5 * n) % 16 for k in range(K)] for n in range(N)])
    d = np.array([[2.0 ** -(b + 3) * (n + 1) for b in range(K // 32)] for n in range(N)],
                 dtype=np.float16)
    W = Q.dequantize("q4_0", {"qs": _pack_nibbles(codes), "d": d})
    for n in range(N):
        for k in range(K):
            assert W[n, k] == 2.0 ** -(k // 32 + 3) * (n + 1) * (((k + 5 * n) % 16) - 8)


def test_q8_0_is_the_signed_code_times_its_block_scale():
    N, K = 3, 64
    codes = np.array([[((7 * k + 3 * n) % 255) - 127 for k in range(K)] for n in range(N)],
                     dtype=np.int8)
    d = np.array([[0.5, 0.25], [1.0, 2.0], [0.125, 4.0]], dtype=np.float16)
    W = Q.dequantize("q8_0", {"qs": codes, "d": d})
    for n in range(N):
        for k in range(K):
            assert W[n, k] == float(d[n, k // 32]) * (((7 * k + 3 * n) % 255) - 127)


def test_q4_k_scale_and_min_reach_exactly_their_sub_block():
    N, K = 1, 512
    codes = np.array([[(3 * k) % 16 for k in range(K)]])
    sm = np.zeros((N, K // 32, 2), dtype=np.uint8)
    for b in range(K // 32):
        sm[0, b] = (b + 1, 63 - 2 * b)
    dm = np.array([[[0.5, 0.25], [0.125, 2.0]]], dtype=np.float16)
    W = Q.dequantize("q4_k", {"qs": _pack_nibbles(codes), "sm": sm, "dm": dm})
    for k in range(K):
        d, dmin = (0.5, 0.25) if k < 256 else (0.125, 2.0)
        b = k // 32
        assert W[0, k] == d * (b + 1) * ((3 * k) % 16) - dmin * (63 - 2 * b)


def test_q6_k_six_bit_codes_and_signed_sub_scales():
    N, K = 2, 256
    codes = np.array([[(k + 11 * n) % 64 for k in range(K)] for n in range(N)])
    ql = _pack_nibbles(codes & 15)
    qh = _pack_crumbs(codes >> 4)
    sc = np.array([[(-1) ** b * (b + 1) + n for b in range(16)] for n in range(N)], dtype=np.int8)
    d = np.array([[0.25], [0.5]], dtype=np.float16)
    W = Q.dequantize("q6_k", {"ql": ql, "qh": qh, "sc": sc, "d": d})
    for n in range(N):
        for k in range(K):
            b = k // 16
            assert W[n, k] == float(d[n, 0]) * ((-1) ** b * (b + 1) + n) * (((k + 11 * n) % 64) - 32)


@pytest.mark.parametrize("fmt", Q.FORMATS)
def test_neutral_codes_give_an_exactly_zero_weight(fmt):
    rng = np.random.default_rng(3)
    N, K = 4, 256
    shp = Q.plane_shapes(fmt, N, K)
    planes = {}
    for name, (dt, shape) in shp.items():
        if dt == np.float16:
            planes[name] = rng.uniform(0.01, 1.0, shape).astype(np.float16)
        else:
            planes[name] = rng.integers(1, 64, shape).astype(dt)
    neutral = {"q8_0": ("qs", 0), "q4_0": ("qs", 0x88), "q6_k": ("ql", 0)}
    if fmt == "q4_k":
        planes["qs"][:] = 0
        planes["sm"][..., 1] = 0
    elif fmt == "q6_k":
        planes["ql"][:] = 0
        planes["qh"][:] = 0b10101010            # q = 32 everywhere
    else:
        name, v = neutral[fmt]
        planes[name][:] = v
    assert np.all(Q.dequantize(fmt, planes) == 0.0)


def test_q4_0_equals_q4_k_with_unit_sub_scales():
    rng = np.random.default_rng(5)
    N, K = 3, 512
    qs = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    e = rng.integers(-12, -2, (N, K // 32))
    d0 = (2.0 ** e).astype(np.float16)                     # powers of two: 8*d exact in fp16
    # q4_k carries one (d, dmin) per 256 elements: make the q4_0 scales equal
    # within each super-block
    d0 = np.repeat(d0[:, ::8], 8, axis=1)
    sm = np.ones((N, K // 32, 2), dtype=np.uint8)
    dm = np.stack([d0[:, ::8], (8 * d0[:, ::8].astype(np.float64)).astype(np.float16)], axis=2)
    a = Q.dequantize("q4_0", {"qs": qs, "d": d0})
    b = Q.dequantize("q4_k", {"qs": qs, "sm": sm, "dm": dm})
    assert np.array_equal(a, b)


def test_q6_k_equals_q8_0_with_shifted_codes():
    rng = np.random.default_rng(6)
    N, K = 2, 256
    codes = rng.integers(0, 64, (N, K))
    sc = rng.integers(-4, 5, (N, K // 16)).astype(np.int8)
    d = (2.0 ** rng.integers(-10, -4, (N, 1))).astype(np.float16)
    # q8_0 blocks are 32 wide: give both 16-element halves one scale first
    sc2 = np.repeat(sc[:, ::2], 2, axis=1)
    W6b = Q.dequantize("q6_k", {"ql": _pack_nibbles(codes & 15), "qh": _pack_crumbs(codes >> 4),
                                "sc": sc2, "d": d})
    d8 = (d.astype(np.float64) * sc2[:, ::2]).astype(np.float16)
    W8 = Q.dequantize("q8_0", {"qs": (codes - 32).astype(np.int8), "d": d8})
    assert np.array_equal(W6b, W8)
