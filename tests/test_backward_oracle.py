"""Pins of the oracle's backward (test infrastructure).

The pages name the backward's kernels (grouped dgrad/wgrad GEMMs, fp32
gradient accumulation fused into the GEMM, deterministic scatter-add;
LongCat-Flash summary, section 5) but print no formulas or values.  The
oracle's backward is the chain rule through the forward with the routing
held fixed; it is pinned to torch's float64 autograd (a library routine) on
the same forward, to the softmax-gradient identity, to the zero-expert
closed form, and to its own sampled-row helper."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def _case(seed=41, T=24, d=64, I=32, N=6, Z=3, k=3, dtype="bf16"):
    cfg = synth.Config("bwd", T=T, d=d, I=I, N=N, Z=Z, k=k, dtype=dtype, seed=seed,
                       bias_lo=-0.01, bias_hi=0.01)
    inp = synth.host_inputs(cfg)
    fwd = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                         inp["W_down"], N, Z, k, dtype)
    dout = synth.host_dout(cfg)
    return cfg, inp, fwd, dout


def _f64(a, dt):
    if a is None:
        return None
    a = synth.bf16_bits_to_f32(a) if dt == "bf16" else np.asarray(a, np.float32)
    return torch.from_numpy(a.astype(np.float64))


def _autograd(cfg, inp, idx, dout, scale=1.0):
    """float64 forward with the routing fixed (gates = scale * p of the
    selected experts), differentiated by torch."""
    dt = cfg.dtype
    x = _f64(inp["x"], dt).requires_grad_()
    wr = _f64(inp["W_router"], dt).requires_grad_()
    wg = _f64(inp["W_gate"], dt).requires_grad_()
    wu = _f64(inp["W_up"], dt).requires_grad_()
    wd = _f64(inp["W_down"], dt).requires_grad_()
    p = torch.softmax(x @ wr.T, dim=1)
    it = torch.from_numpy(idx.astype(np.int64))
    gate = scale * p.gather(1, it)
    rows = []
    for t in range(cfg.T):
        o = torch.zeros(cfg.d, dtype=torch.float64)
        for j in range(cfg.k):
            e = int(idx[t, j])
            if e >= cfg.N:
                o = o + gate[t, j] * x[t]
            else:
                h = torch.nn.functional.silu(wg[e] @ x[t]) * (wu[e] @ x[t])
                o = o + gate[t, j] * (wd[e] @ h)
        rows.append(o)
    out = torch.stack(rows)
    out.backward(_f64(dout, dt))
    return {"dx": x.grad, "dw_router": wr.grad, "dw_gate": wg.grad, "dw_up": wu.grad,
            "dw_down": wd.grad}


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("dt,scale", [("bf16", 1.0), ("f32", 1.0), ("bf16", 2.5)])
def test_backward_matches_float64_autograd(dt, scale):
    """With a routed scale s != 1 the gates are s * p, so the router gradient
    carries s (catches dp = dgate where dp = s * dgate is due)."""
    cfg, inp, fwd, dout = _case(dtype=dt)
    assert (fwd["idx"] >= cfg.N).any() and (fwd["idx"] < cfg.N).any()
    gate = (np.float32(scale) * fwd["gate"]).astype(np.float32)
    r = oracle.backward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"],
                        fwd["idx"], gate, synth.bf16_bits_to_f32(dout) if dt == "bf16"
                        else dout, cfg.N, cfg.Z, dt, routed_scale=scale)
    ref = _autograd(cfg, inp, fwd["idx"], dout, scale)
    for key in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down"):
        err = _rel(r[key], ref[key].numpy())
        assert err < 2e-5, (key, err)


def test_weight_gradients_accumulate():
    cfg, inp, fwd, dout = _case(seed=42)
    df = synth.bf16_bits_to_f32(dout)
    args = (inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"], fwd["idx"],
            fwd["gate"], df, cfg.N, cfg.Z, "bf16")
    fresh = oracle.backward(*args)
    rng = np.random.default_rng(0)
    prior = {k: rng.standard_normal(fresh[k].shape).astype(np.float32)
             for k in ("dw_router", "dw_gate", "dw_up", "dw_down")}
    acc = oracle.backward(*args, grads={k: v.copy() for k, v in prior.items()})
    for key, v in prior.items():
        assert _rel(acc[key] - v, fresh[key]) < 1e-5, key
    assert np.array_equal(acc["dx"], fresh["dx"])


def test_router_gradient_columns_sum_to_zero():
    """sum_e dl[t, e] = 0 for a softmax, so every column of dW_router sums to
    ~0 (a dropped <p, dp> term or a gradient through the logit instead of p
    breaks it)."""
    cfg, inp, fwd, dout = _case(seed=43)
    r = oracle.backward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"],
                        fwd["idx"], fwd["gate"], synth.bf16_bits_to_f32(dout), cfg.N, cfg.Z,
                        "bf16")
    col = r["dw_router"].sum(0)
    assert np.abs(col).max() < 1e-5 * np.abs(r["dw_router"]).sum(0).max()
    assert np.abs(r["dw_router"]).max() > 0


def test_all_zero_routing_closed_form():
    """Every slot on a zero expert: expert gradients stay zero, dgate = <dout, x>
    and dx = zsum * dout + W_router^T dl."""
    cfg, inp, _, dout = _case(seed=44)
    b = np.zeros(cfg.E, np.float32)
    b[cfg.N:] = 10.0
    fwd = oracle.forward(inp["x"], inp["W_router"], b, inp["W_gate"], inp["W_up"], inp["W_down"],
                         cfg.N, cfg.Z, cfg.k, "bf16")
    assert (fwd["idx"] >= cfg.N).all()
    df = synth.bf16_bits_to_f32(dout)
    r = oracle.backward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"],
                        fwd["idx"], fwd["gate"], df, cfg.N, cfg.Z, "bf16")
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert not r[key].any()
    x = synth.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    wr = synth.bf16_bits_to_f32(inp["W_router"]).astype(np.float64)
    p = np.exp(x @ wr.T - (x @ wr.T).max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dp = np.zeros_like(p)
    for t in range(cfg.T):
        for j in range(cfg.k):
            dp[t, fwd["idx"][t, j]] = df[t] @ x[t]
    dl = p * (dp - (p * dp).sum(1, keepdims=True))
    zs = fwd["gate"].astype(np.float64).sum(1)
    ref = zs[:, None] * df + dl @ wr
    assert _rel(r["dx"], ref) < 1e-5


def test_token_backward_and_wgrad_rows_agree_with_the_whole_backward():
    cfg, inp, fwd, dout = _case(seed=45)
    df = synth.bf16_bits_to_f32(dout)
    r = oracle.backward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"],
                        fwd["idx"], fwd["gate"], df, cfg.N, cfg.Z, "bf16")
    experts = {e: (inp["W_gate"][e], inp["W_up"][e], inp["W_down"][e]) for e in range(cfg.N)}
    for t in (0, 7, cfg.T - 1):
        tb = oracle.token_backward(inp["x"][t], "bf16", inp["W_router"], cfg.N, fwd["idx"][t],
                                   fwd["gate"][t], df[t], experts)
        assert np.array_equal(tb["dx"], r["dx"][t])
    for e in range(cfg.N):
        sel = [(t, j) for t in range(cfg.T) for j in range(cfg.k) if fwd["idx"][t, j] == e]
        if not sel:
            continue
        ts = [t for t, _ in sel]
        gates = np.array([fwd["gate"][t, j] for t, j in sel], np.float32)
        for row in (0, cfg.I - 1):
            w = oracle.expert_wgrad_row(inp["x"][ts], "bf16", df[ts], gates, *experts[e], row)
            assert np.array_equal(w["dw_gate_row"], r["dw_gate"][e, row])
            assert np.array_equal(w["dw_up_row"], r["dw_up"][e, row])
            assert np.array_equal(w["dw_down_col"], r["dw_down"][e, :, row])
