"""Pins of the CPU oracle to things other than itself (CPU only).

Each test names the plausible mistake it would catch.  The passages the
oracle follows are cited in oracle/oracle.c; the model-size arithmetic uses
the numbers printed on the LongCat-Flash summary page (tests/golden).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

U32 = 2.0 ** -24  # fp32 unit roundoff


def _inputs(cfg):
    return synth.host_inputs(cfg)


def _f(a, dt):
    return synth.bf16_bits_to_f32(a) if dt == "bf16" else np.asarray(a, dtype=np.float32)


SMALLISH = synth.Config("pin", T=37, d=48, I=20, N=6, Z=3, k=4, dtype="f32", seed=11)


# ---------------------------------------------------------------- logits ---
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_logits_match_float64_matmul(dt):
    """Catches a transposed router operand or a wrong row stride."""
    cfg = SMALLISH.with_(dtype=dt, d=96, N=9, Z=5)
    x, wr = synth.host_x(cfg), synth.host_router(cfg)
    xf, wf = _f(x, dt).astype(np.float64), _f(wr, dt).astype(np.float64)
    got = oracle.router_logits(x, wr, dt).astype(np.float64)
    ref = xf @ wf.T
    bound = cfg.d * U32 / (1 - cfg.d * U32) * (np.abs(xf) @ np.abs(wf).T) + 1e-30
    assert (np.abs(got - ref) <= bound).all()


# --------------------------------------------------------------- softmax ---
def test_softmax_is_a_distribution_and_matches_float64():
    """Catches a softmax over the FFN experts only, or a missing max shift."""
    rng = np.random.default_rng(0)
    E = 23
    logits = (rng.standard_normal((50, E)) * 3).astype(np.float32)
    logits[0] += 80.0  # would overflow expf without the max shift
    _, _, _, p = oracle.route_from_logits(logits, np.zeros(E, np.float32), 3)
    assert (p > 0).all()
    assert np.abs(p.astype(np.float64).sum(1) - 1.0).max() <= 4 * E * U32
    l64 = logits.astype(np.float64)
    ref = np.exp(l64 - l64.max(1, keepdims=True))
    ref /= ref.sum(1, keepdims=True)
    assert np.abs(p - ref).max() <= 1e-6 * ref.max()
    assert (np.abs(p - ref) <= 16 * U32 * ref + 1e-12).all()


# ----------------------------------------------------------------- top-k ---
def _brute_topk(s, k):
    """Full sort by (score descending, index ascending)."""
    order = sorted(range(len(s)), key=lambda e: (-float(s[e]), e))
    return order


@pytest.mark.parametrize("k", [1, 3, 7, 12])
def test_topk_matches_brute_force_with_ties(k):
    """Catches a wrong tie-break, an off-by-one in k or a wrong margin."""
    rng = np.random.default_rng(k)
    E, T = 12, 40
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)  # many equal logits
    bias = rng.choice(np.array([0.0, 0.01, -0.01], np.float32), size=E)
    idx, gate, margin, p = oracle.route_from_logits(logits, bias, k)
    s = (p + bias).astype(np.float32)  # the fp32 sum the oracle selects on
    for t in range(T):
        order = _brute_topk(s[t], k)
        assert list(idx[t]) == order[:k]
        if k < E:
            assert margin[t] == np.float32(s[t, order[k - 1]] - s[t, order[k]])
        else:
            assert math.isinf(margin[t])
        assert (gate[t] == p[t, idx[t]]).all()  # gate = unbiased probability, bit for bit


def test_bias_enters_probabilities_not_logits():
    """Worked example, checkable by hand.  p = (0.5, 0.3, 0.2), bias (0, 0, 0.15):
    p + b = (0.5, 0.3, 0.35) selects experts {0, 2}; adding the bias to the
    logits instead would scale p_2 by e^0.15 to 0.232 < 0.3 and select {0, 1}.
    Gates stay the unbiased 0.5 and 0.2 (no renormalisation)."""
    logits = np.log(np.array([[0.5, 0.3, 0.2]], np.float64)).astype(np.float32)
    idx, gate, _, _ = oracle.route_from_logits(logits, np.array([0, 0, 0.15], np.float32), 2)
    assert list(idx[0]) == [0, 2]
    assert np.allclose(gate[0], [0.5, 0.2], rtol=1e-6)

    # and the whole forward on it: N=2 FFN experts, Z=1, d=1, I=1, x=2;
    # expert 0: W_gate=1, W_up=0.5, W_down=3 -> y = 3 * silu(2) * 1
    x = np.array([[2.0]], np.float32)
    wg = np.array([[[1.0]], [[7.0]]], np.float32)
    wu = np.array([[[0.5]], [[7.0]]], np.float32)
    wd = np.array([[[3.0]], [[7.0]]], np.float32)
    out = oracle.combine_given_routing(x, "f32", 2, idx, gate, wg, wu, wd)
    silu2 = 2.0 / (1.0 + math.exp(-2.0))
    expect = 0.2 * 2.0 + 0.5 * (3.0 * silu2 * 1.0)
    assert abs(out[0, 0] - expect) <= 1e-6 * expect


def test_k_equals_E_selects_everything():
    cfg = SMALLISH.with_(k=SMALLISH.N + SMALLISH.Z)
    inp = _inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, cfg.Z, cfg.k, cfg.dtype)
    assert (r["counts"] == cfg.T).all()
    assert all(sorted(row) == list(range(cfg.E)) for row in r["idx"])
    assert np.isinf(r["margin"]).all()


def test_forced_set_and_gates_independent_of_bias():
    """A +10 bias on a set S of k experts selects exactly S for every token;
    the gates do not move when the bias elsewhere changes (catches gates taken
    from the biased score)."""
    cfg = SMALLISH
    inp = _inputs(cfg)
    logits = oracle.router_logits(inp["x"], inp["W_router"], cfg.dtype)
    S = [1, 4, 6, 8]
    b1 = np.zeros(cfg.E, np.float32)
    b1[S] = 10.0
    b2 = b1.copy()
    b2[[0, 2, 3]] = [0.3, -0.2, 0.05]
    i1, g1, _, p = oracle.route_from_logits(logits, b1, cfg.k)
    i2, g2, _, _ = oracle.route_from_logits(logits, b2, cfg.k)
    assert all(sorted(r) == S for r in i1)
    assert (i1 == i2).all() and (g1 == g2).all()
    for t in range(cfg.T):  # within S the order is by probability
        assert (np.diff(p[t, i1[t]]) <= 0).all()


def test_counts_sum_and_recount():
    cfg = SMALLISH.with_(T=300, k=5)
    inp = _inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, cfg.Z, cfg.k, cfg.dtype)
    assert r["counts"].sum() == cfg.T * cfg.k
    assert (r["counts"] == np.bincount(r["idx"].ravel(), minlength=cfg.E)).all()
    nffn = (r["idx"] < cfg.N).sum(1)
    assert nffn.min() >= 0 and nffn.max() <= min(cfg.k, cfg.N)
    assert all(len(set(row)) == cfg.k for row in r["idx"])


# ------------------------------------------------------------- FFN expert ---
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_single_expert_matches_float64_swiglu(dt):
    """N=1, Z=0, k=1: the softmax gate is exactly 1 and out = W_down(silu(W_gate x)*(W_up x)).
    d != I catches a transposed W_down; the float64 reference catches a wrong
    silu sign or a swapped gate/up."""
    torch = pytest.importorskip("torch")
    cfg = synth.Config("one", T=5, d=40, I=24, N=1, Z=0, k=1, dtype=dt, seed=5)
    inp = _inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, cfg.Z, cfg.k, dt)
    assert (r["gate"] == 1.0).all()
    X = torch.from_numpy(_f(inp["x"], dt).astype(np.float64))
    Wg = torch.from_numpy(_f(inp["W_gate"], dt)[0].astype(np.float64))
    Wu = torch.from_numpy(_f(inp["W_up"], dt)[0].astype(np.float64))
    Wd = torch.from_numpy(_f(inp["W_down"], dt)[0].astype(np.float64))
    ref = (torch.nn.functional.silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    err = np.abs(r["out"] - ref.numpy()).max() / np.abs(ref.numpy()).max()
    assert err < 2e-6


def test_linear_in_w_down_exactly():
    """Doubling W_down doubles every product and partial sum exactly."""
    cfg = synth.Config("one", T=6, d=32, I=16, N=1, Z=0, k=1, dtype="f32", seed=2)
    inp = _inputs(cfg)
    args = (inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"])
    a = oracle.forward(*args, inp["W_down"], 1, 0, 1, "f32")["out"]
    b = oracle.forward(*args, 2 * inp["W_down"], 1, 0, 1, "f32")["out"]
    assert (b == 2 * a).all()


def test_w_up_zero_leaves_only_the_zero_experts():
    """W_up = 0 kills every FFN term; out must be exactly zsum * x (catches a
    dropped or double-counted zero-expert term)."""
    cfg = SMALLISH
    inp = _inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"],
                       np.zeros_like(inp["W_up"]), inp["W_down"], cfg.N, cfg.Z, cfg.k, cfg.dtype)
    for t in range(cfg.T):
        z = np.float32(0)
        for j in range(cfg.k):
            if r["idx"][t, j] >= cfg.N:
                z = np.float32(z + r["gate"][t, j])
        assert (r["out"][t] == z * inp["x"][t]).all()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_all_zero_routing_returns_gate_sum_times_x(dt):
    """Bias +10 on the zero experts (Z >= k): every slot is a zero expert, so
    out = (sum of gates) * x up to the one fp32 rounding of the product.  FFN
    weights are NaN: touching them would poison the output."""
    cfg = SMALLISH.with_(dtype=dt, Z=5)
    inp = _inputs(cfg)
    b = np.zeros(cfg.E, np.float32)
    b[cfg.N:] = 10.0
    nan = np.float32("nan")
    if dt == "f32":
        wg = np.full_like(inp["W_gate"], nan)
    else:
        wg = np.full_like(inp["W_gate"], 0x7FC0)  # bfloat16 quiet NaN
    r = oracle.forward(inp["x"], inp["W_router"], b, wg, wg, wg, cfg.N, cfg.Z, cfg.k, dt)
    assert (r["idx"] >= cfg.N).all()
    xf = _f(inp["x"], dt)
    for t in range(cfg.T):
        z = np.float32(0)
        for j in range(cfg.k):
            z = np.float32(z + r["gate"][t, j])
        assert (r["out"][t] == z * xf[t]).all()
        assert abs(float(z) - float(np.sum(r["gate"][t], dtype=np.float64))) < 1e-6


def test_no_ffn_experts():
    cfg = synth.Config("n0", T=9, d=16, I=8, N=0, Z=4, k=2, dtype="f32", seed=1)
    x, wr, b = synth.host_x(cfg), synth.host_router(cfg), synth.host_bias(cfg)
    r = oracle.forward(x, wr, b, None, None, None, 0, 4, 2, "f32")
    zs = (r["gate"][:, 0] + r["gate"][:, 1]).astype(np.float32)
    assert (r["out"] == zs[:, None] * x).all()


def test_z0_reduces_to_textbook_topk_softmax_moe():
    """Z = 0: dense-masked float64 top-k softmax MoE (no renormalisation)."""
    cfg = synth.Config("z0", T=50, d=32, I=12, N=7, Z=0, k=3, dtype="f32", seed=3,
                       bias_lo=-0.05, bias_hi=0.05)
    inp = _inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, 0, cfg.k, "f32")
    X = inp["x"].astype(np.float64)
    L = X @ inp["W_router"].astype(np.float64).T
    P = np.exp(L - L.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    S = P + inp["bias"].astype(np.float64)
    Y = []
    for e in range(cfg.N):
        G = X @ inp["W_gate"][e].astype(np.float64).T
        U = X @ inp["W_up"][e].astype(np.float64).T
        Y.append((G / (1 + np.exp(-G)) * U) @ inp["W_down"][e].astype(np.float64).T)
    Y = np.stack(Y)  # [N, T, d]
    checked = 0
    for t in range(cfg.T):
        order = np.argsort(-S[t], kind="stable")
        if S[t, order[cfg.k - 1]] - S[t, order[cfg.k]] < 1e-6:
            continue
        checked += 1
        assert sorted(order[: cfg.k]) == sorted(r["idx"][t])
        mask = np.zeros(cfg.N)
        mask[order[: cfg.k]] = 1
        ref = (mask * P[t]) @ Y[:, t, :]
        assert np.abs(r["out"][t] - ref).max() <= 1e-5 * max(1e-3, np.abs(ref).max())
    assert checked > 40


def test_identical_experts_closed_form():
    """All N experts share weights: out = (sum of FFN gates) FFN(x) + zsum x."""
    cfg = SMALLISH.with_(dtype="f32")
    inp = _inputs(cfg)
    wg = np.repeat(inp["W_gate"][:1], cfg.N, 0)
    wu = np.repeat(inp["W_up"][:1], cfg.N, 0)
    wd = np.repeat(inp["W_down"][:1], cfg.N, 0)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], wg, wu, wd, cfg.N, cfg.Z, cfg.k,
                       "f32")
    X = inp["x"].astype(np.float64)
    G, U = X @ wg[0].astype(np.float64).T, X @ wu[0].astype(np.float64).T
    F = (G / (1 + np.exp(-G)) * U) @ wd[0].astype(np.float64).T
    ffn = r["idx"] < cfg.N
    gf = (r["gate"] * ffn).sum(1, dtype=np.float64)
    gz = (r["gate"] * ~ffn).sum(1, dtype=np.float64)
    ref = gf[:, None] * F + gz[:, None] * X
    assert np.abs(r["out"] - ref).max() <= 1e-5 * np.abs(ref).max()


def test_token_permutation_equivariance_and_determinism():
    cfg = SMALLISH.with_(T=64, dtype="bf16")
    inp = _inputs(cfg)
    args = (inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
            cfg.N, cfg.Z, cfg.k, "bf16")
    a = oracle.forward(inp["x"], *args)
    a2 = oracle.forward(inp["x"], *args)
    assert (a["out"] == a2["out"]).all() and (a["idx"] == a2["idx"]).all()
    perm = np.random.default_rng(1).permutation(cfg.T)
    b = oracle.forward(inp["x"][perm], *args)
    assert (b["out"] == a["out"][perm]).all()
    assert (b["idx"] == a["idx"][perm]).all() and (b["counts"] == a["counts"]).all()


def test_token_output_matches_full_forward():
    cfg = SMALLISH.with_(dtype="bf16")
    inp = _inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, cfg.Z, cfg.k, "bf16")
    for t in (0, 13, cfg.T - 1):
        ex = {int(e): (inp["W_gate"][e], inp["W_up"][e], inp["W_down"][e])
              for e in r["idx"][t] if e < cfg.N}
        o = oracle.token_output(inp["x"][t], "bf16", cfg.N, r["idx"][t], r["gate"][t], ex)
        assert (o == r["out"][t]).all()


# ---------------------------------------------------------- routed scale ---
def test_routed_scale_of_two_doubles_gates_and_output_exactly():
    """gate = s * p for every selected slot (FFN and zero), selection
    unchanged.  With s = 2 every fp32 operation of the combine scales
    exactly, so the output is exactly twice the unscaled one (catches a scale
    applied to FFN slots only, or to the selection)."""
    cfg = SMALLISH.with_(dtype="bf16", T=41)
    inp = _inputs(cfg)
    a = (inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
         cfg.N, cfg.Z, cfg.k, "bf16")
    r1 = oracle.forward(*a)
    r2 = oracle.forward(*a, routed_scale=2.0)
    assert (r1["idx"] >= cfg.N).any() and (r1["idx"] < cfg.N).any()
    assert np.array_equal(r1["idx"], r2["idx"]) and np.array_equal(r1["counts"], r2["counts"])
    assert np.array_equal(r2["gate"], 2.0 * r1["gate"])
    assert np.array_equal(r2["out"], 2.0 * r1["out"])
    assert np.array_equal(oracle.forward(*a, routed_scale=1.0)["out"], r1["out"])


def test_routed_scale_matches_float64():
    """s = 2.5: gates and output against a float64 evaluation with the
    oracle's own routing."""
    cfg = SMALLISH.with_(dtype="f32", T=29)
    inp = _inputs(cfg)
    s = 2.5
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, cfg.Z, cfg.k, "f32", routed_scale=s)
    x = inp["x"].astype(np.float64)
    l = x @ inp["W_router"].astype(np.float64).T
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    g = s * np.take_along_axis(p, r["idx"].astype(np.int64), 1)
    assert np.abs(r["gate"] - g).max() <= 1e-6 * g.max()
    ref = np.zeros_like(x)
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = int(r["idx"][t, j])
            if e >= cfg.N:
                ref[t] += g[t, j] * x[t]
            else:
                wg, wu, wd = (inp[w][e].astype(np.float64) for w in ("W_gate", "W_up", "W_down"))
                gg, uu = wg @ x[t], wu @ x[t]
                ref[t] += g[t, j] * (wd @ (gg / (1 + np.exp(-gg)) * uu))
    assert np.linalg.norm(r["out"] - ref) / np.linalg.norm(ref) < 1e-5


# ------------------------------------- expert-streamed pieces of the same ---
def _slot_outputs(cfg, inp, idx, mats_of):
    """y [T, k, d] of every FFN slot through oracle.ffn_pairs (zero slots NaN,
    so a combine that read them would not stay finite)."""
    y = np.full((cfg.T, cfg.k, cfg.d), np.nan, np.float32)
    pairs = [(t, j) for t in range(cfg.T) for j in range(cfg.k) if idx[t, j] < cfg.N]
    yy = oracle.ffn_pairs([inp["x"][t] for t, _ in pairs], cfg.dtype,
                          [mats_of(int(idx[t, j])) for t, j in pairs])
    for (t, j), row in zip(pairs, yy):
        y[t, j] = row
    return y


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ffn_pairs_and_combine_slots_reproduce_the_forward_bit_for_bit(dt):
    """The expert-major split used by the full-size checks (one expert's
    matrices in memory at a time) is the same arithmetic as the token-major
    forward: catches a slot order or a zero-slot term that differs."""
    cfg = SMALLISH.with_(dtype=dt, T=53)
    inp = _inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, cfg.Z, cfg.k, dt)
    y = _slot_outputs(cfg, inp, r["idx"],
                      lambda e: (inp["W_gate"][e], inp["W_up"][e], inp["W_down"][e]))
    out = oracle.combine_slots(inp["x"], dt, cfg.N, r["idx"], r["gate"], y)
    assert np.array_equal(out, r["out"])


def test_combine_slots_matches_float64_formula():
    """out = (sum of zero-slot gates) x + sum_j gate_j y_j, against a float64
    evaluation of the formula with arbitrary slot outputs: catches a dropped
    zero-expert term, a gate applied to the wrong slot or a zero slot's row
    being read."""
    rng = np.random.default_rng(5)
    T, k, d, N = 31, 5, 24, 6
    x = rng.standard_normal((T, d)).astype(np.float32)
    idx = np.stack([rng.permutation(N + 4)[:k] for _ in range(T)]).astype(np.int32)
    gate = rng.random((T, k)).astype(np.float32)
    y = rng.standard_normal((T, k, d)).astype(np.float32)
    y[idx >= N] = np.nan
    got = oracle.combine_slots(x, "f32", N, idx, gate, y)
    ffn = idx < N
    g64 = gate.astype(np.float64)
    zs = np.where(~ffn, g64, 0).sum(1)
    ref = zs[:, None] * x + np.einsum("tk,tkd->td", np.where(ffn, g64, 0),
                                      np.where(ffn[..., None], y, 0).astype(np.float64))
    bound = (k + 2) * U32 * (np.abs(zs)[:, None] * np.abs(x) +
                             np.einsum("tk,tkd->td", np.where(ffn, g64, 0),
                                       np.abs(np.where(ffn[..., None], y, 0)))) + 1e-30
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= bound).all()


# -------------------------------------------------- the pages' arithmetic ---
def test_three_matrix_experts_match_the_activated_parameter_range():
    """The activated-parameter range printed on the page (18.6B .. 31.3B, i.e.
    0 .. 12 FFN experts per token over 28 layers) equals 12 three-matrix d x I
    experts per layer; a two-matrix expert would give 8.45B."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_model_config.json")))
    per = g["hidden_size"] * g["ffn_expert_width"]
    span = g["activated_params_max_B"] - g["activated_params_min_B"]
    three = g["layers_excluding_mtp"] * g["experts_per_token"] * 3 * per / 1e9
    two = g["layers_excluding_mtp"] * g["experts_per_token"] * 2 * per / 1e9
    assert abs(three - span) < 0.1
    assert abs(two - span) > 4
    # the mean of ~27B activated implies ~7.95 FFN experts per token
    mean_ffn = (g["activated_params_mean_B"] - g["activated_params_min_B"]) / (three / 12)
    assert g["ffn_experts_per_token_min_benchmark"] <= mean_ffn <= g["ffn_experts_per_token_max_benchmark"]
