"""GPU parity of the block's backward (moe_zc_backward through the C ABI)
against the CPU oracle's backward.  The routing given to both sides is the
oracle's own forward routing, so no input of the oracle comes from the GPU.
Tolerances: bf16 operands and intermediates (G, U, dG, dU, H, dl and the
permuted dx rows are rounded to bfloat16), fp32 accumulation; every output
tensor within 2e-2 relative Frobenius error of the oracle (the forward's
bound), every dx row within 1.5x of that."""
import os

import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("zero_computation_expert_amd")

TOL = 2e-2
DEV = "cuda:0"


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def case(seed, T, d, I, N, Z, k, bias=None):
    cfg = synth.Config("bwd", T=T, d=d, I=I, N=N, Z=Z, k=k, dtype="bf16", seed=seed,
                       bias_lo=-0.01, bias_hi=0.01)
    inp = synth.host_inputs(cfg)
    if bias is not None:
        inp["bias"] = bias.astype(np.float32)
    logits = oracle.router_logits(inp["x"], inp["W_router"], "bf16")
    idx, gate, _, _ = oracle.route_from_logits(logits, inp["bias"], k)
    return cfg, inp, idx, gate, synth.host_dout(cfg)


def run_gpu(cfg, inp, idx, gate, dout, prior=None, poison=False, scale=1.0):
    N = cfg.N
    w = {key: (dev_bf16(inp[key]) if N > 0 else None) for key in ("W_gate", "W_up", "W_down")}
    grads = {}
    if prior is not None:
        grads = {key: dev(v) for key, v in prior.items()}
    ws = None
    if poison:
        nb = moe.backward_workspace_bytes(cfg.T, cfg.d, cfg.I, cfg.N, cfg.Z, cfg.k)
        ws = torch.full((max(nb, 1),), 0xFF, dtype=torch.uint8, device=DEV)  # NaN bytes
    dx, dwr, dwg, dwu, dwd = moe.backward(
        dev_bf16(inp["x"]), dev_bf16(inp["W_router"]), w["W_gate"], w["W_up"], w["W_down"],
        dev(idx.astype(np.int32)), dev(gate.astype(np.float32)), dev_bf16(dout), N, cfg.Z,
        dW_router=grads.get("dw_router"), dW_gate=grads.get("dw_gate"),
        dW_up=grads.get("dw_up"), dW_down=grads.get("dw_down"), workspace=ws, routed_scale=scale)
    torch.cuda.synchronize()
    out = {"dx": synth.bf16_bits_to_f32(P.to_np(dx)), "dw_router": P.to_np(dwr)}
    if N > 0:
        out.update({"dw_gate": P.to_np(dwg), "dw_up": P.to_np(dwu), "dw_down": P.to_np(dwd)})
    return out


def ref_backward(cfg, inp, idx, gate, dout, scale=1.0):
    return oracle.backward(inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"],
                           idx, gate, synth.bf16_bits_to_f32(dout), cfg.N, cfg.Z, "bf16",
                           routed_scale=scale)


def compare(got, ref, keys=("dx", "dw_router", "dw_gate", "dw_up", "dw_down")):
    errs = {}
    for key in keys:
        g, r = got[key], ref[key]
        assert np.isfinite(g).all(), f"{key}: non-finite values"
        errs[key] = P.rel_frob(g, r)
    print("[bwd parity] " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, (key, e)
    worst = P.worst_token_rel(got["dx"], ref["dx"])
    assert worst <= 1.5 * TOL, worst
    return errs


@pytest.mark.parametrize("shape", [
    # (seed, T, d, I, N, Z, k): ragged I (not a multiple of 256), several
    # chunks per expert, E not a multiple of 8 (padded router-gradient rows)
    (51, 200, 256, 192, 12, 6, 4),
    (52, 64, 128, 64, 8, 4, 2),
    (53, 300, 384, 320, 5, 6, 3),
    (54, 512, 256, 128, 4, 2, 4),
    # d and I not multiples of 64: K tails in every transposed-read operand
    # and partial 32-column sub-tiles in the wgrad outputs
    (60, 150, 200, 72, 6, 3, 3),
    (61, 97, 136, 40, 3, 5, 2),
])
def test_backward_parity(shape):
    seed, T, d, I, N, Z, k = shape
    cfg, inp, idx, gate, dout = case(seed, T, d, I, N, Z, k)
    print(f"[bwd] T={T} d={d} I={I} N={N} Z={Z} k={k}", flush=True)
    compare(run_gpu(cfg, inp, idx, gate, dout, poison=True), ref_backward(cfg, inp, idx, gate, dout))


def test_backward_routed_scale():
    """Gates scaled by 2.5 (as the forward with routed_scale 2.5 gives them):
    the router gradient carries the scale; every gradient against the
    oracle's backward with the same scale."""
    s = 2.5
    cfg, inp, idx, gate, dout = case(62, 200, 256, 192, 12, 6, 4)
    gs = (np.float32(s) * gate).astype(np.float32)
    compare(run_gpu(cfg, inp, idx, gs, dout, poison=True, scale=s),
            ref_backward(cfg, inp, idx, gs, dout, scale=s))


@pytest.mark.parametrize("T", [700, 1500])
def test_backward_hot_expert_long_k(T):
    """One expert takes every token: its wgrad reduces over T rows (11 or
    24 K-steps through the three-buffer ring) and its dgrad spans 5 or 10
    chunks (above 8, tiles go in groups of 8 chunks per row block)."""
    N, Z = 6, 3
    b = np.zeros(N + Z, np.float32)
    b[2] = 10.0
    cfg, inp, idx, gate, dout = case(55, T, 256, 128, N, Z, 3, bias=b)
    assert (idx == 2).any(1).all()
    compare(run_gpu(cfg, inp, idx, gate, dout), ref_backward(cfg, inp, idx, gate, dout))


def test_backward_accumulates_into_weight_gradients():
    cfg, inp, idx, gate, dout = case(56, 128, 128, 64, 6, 3, 3)
    rng = np.random.default_rng(1)
    prior = {"dw_router": rng.standard_normal((cfg.E, cfg.d)).astype(np.float32),
             "dw_gate": rng.standard_normal((cfg.N, cfg.I, cfg.d)).astype(np.float32),
             "dw_up": rng.standard_normal((cfg.N, cfg.I, cfg.d)).astype(np.float32),
             "dw_down": rng.standard_normal((cfg.N, cfg.d, cfg.I)).astype(np.float32)}
    # an expert no token selects keeps its prior gradient bit for bit
    got = run_gpu(cfg, inp, idx, gate, dout, prior=prior)
    ref = ref_backward(cfg, inp, idx, gate, dout)
    used = np.zeros(cfg.N, bool)
    used[idx[idx < cfg.N]] = True
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(got[key][~used], prior[key][~used])
        got[key] = got[key] - prior[key]
    got["dw_router"] = got["dw_router"] - prior["dw_router"]
    compare(got, ref)


def test_backward_all_zero_routing():
    """Every slot on a zero expert: the expert gradients stay untouched and
    dx = zsum * dout + W_router^T dl."""
    N, Z = 6, 5
    b = np.zeros(N + Z, np.float32)
    b[N:] = 10.0
    cfg, inp, idx, gate, dout = case(57, 96, 128, 64, N, Z, 4, bias=b)
    assert (idx >= N).all()
    got = run_gpu(cfg, inp, idx, gate, dout)
    ref = ref_backward(cfg, inp, idx, gate, dout)
    for key in ("dw_gate", "dw_up", "dw_down"):
        assert not got[key].any(), key
    compare(got, ref, keys=("dx", "dw_router"))


def test_backward_no_ffn_experts():
    cfg, inp, idx, gate, dout = case(58, 80, 128, 64, 0, 7, 3)
    got = run_gpu(cfg, inp, idx, gate, dout)
    ref = ref_backward(cfg, inp, idx, gate, dout)
    compare(got, ref, keys=("dx", "dw_router"))


def test_backward_is_deterministic_and_ignores_invalid_slots():
    cfg, inp, idx, gate, dout = case(59, 160, 128, 64, 8, 4, 3)
    a = run_gpu(cfg, inp, idx, gate, dout)
    b = run_gpu(cfg, inp, idx, gate, dout)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    # an out-of-range entry and a repeated expert are ignored: every other
    # token's dx is unchanged bit for bit (a token's dx depends on its own
    # slots only)
    bad = idx.copy()
    bad[5, 1] = cfg.E + 3
    bad[9, 2] = bad[9, 0]
    c = run_gpu(cfg, inp, bad, gate, dout)
    keep = np.ones(cfg.T, bool)
    keep[[5, 9]] = False
    assert np.array_equal(c["dx"][keep], a["dx"][keep])
    assert np.isfinite(c["dx"]).all()


def test_backward_prod_full_size_sparse_dout():
    """The production shape (T=8192, d=6144, I=2048, 512 + 256 experts,
    top-12) with the oracle's routing, and an output gradient that is zero
    except on 24 sampled tokens.  Every token still runs through every
    kernel, but only the sampled ones contribute, so the oracle's per-token
    backward of those 24 tokens determines every gradient:
      - dx of the sampled tokens, one by one; dx of all others exactly zero;
      - the whole router weight gradient dW_router [768, 6144] (the oracle's
        router-logit gradients of the sampled tokens times their x rows);
      - the whole weight gradients of four experts the samples use, and
        exactly zero gradients for every expert they do not use."""
    import concurrent.futures as cf
    import time

    t0 = time.time()
    log = lambda m: print(f"[bwd prod] {m} ({time.time() - t0:.0f}s)", flush=True)  # noqa: E731
    cfg = synth.PROD
    x = synth.host_x(cfg)
    wr = synth.host_router(cfg)
    bias = synth.host_bias(cfg)
    logits = oracle.router_logits(x, wr, "bf16")
    idx, gate, _, _ = oracle.route_from_logits(logits, bias, cfg.k)
    rng = np.random.default_rng(7)
    S = np.array(sorted(set(rng.choice(cfg.T, 22, replace=False).tolist()) | {0, cfg.T - 1}))
    dinp = synth.device_inputs(cfg)
    dout_d = synth.device_dout(cfg)
    keep = torch.zeros(cfg.T, dtype=torch.bool, device=DEV)
    keep[torch.from_numpy(S).to(DEV)] = True
    dout_d[~keep] = 0
    dx, dwr, dwg, dwu, dwd = moe.backward(dinp["x"], dinp["W_router"], dinp["W_gate"],
                                          dinp["W_up"], dinp["W_down"], dev(idx),
                                          dev(gate), dout_d, cfg.N, cfg.Z)
    torch.cuda.synchronize()
    log(f"GPU backward done; {len(S)} tokens carry a gradient")
    dout = synth.bf16_bits_to_f32(synth.host_dout(cfg))
    dx_h = synth.bf16_bits_to_f32(P.to_np(dx))
    used = sorted({int(e) for t in S for e in idx[t] if e < cfg.N})
    mats = {e: tuple(P.to_np(dinp["W_" + w][e]) for w in ("gate", "up", "down")) for e in used}
    log(f"{len(used)} experts copied to the host")

    def one(t):
        return oracle.token_backward(x[t], "bf16", wr, cfg.N, idx[t], gate[t], dout[t],
                                     {int(e): mats[int(e)] for e in idx[t] if e < cfg.N})

    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        tb = dict(zip(S.tolist(), ex.map(one, S.tolist())))
    log("oracle per-token backward done")
    # dx
    for t in S:
        err = P.rel_frob(dx_h[t], tb[t]["dx"])
        assert err <= 1.5 * TOL, (t, err)
    other = np.ones(cfg.T, bool)
    other[S] = False
    assert not dx_h[other].any(), "dx of a token with zero output gradient is not zero"
    err = P.rel_frob(dx_h[S], np.stack([tb[t]["dx"] for t in S]))
    log(f"dx of the sampled tokens rel err {err:.3e}; all others exactly zero")
    assert err <= TOL
    # dW_router = sum over the sampled tokens of dl_t x_t^T
    xf = synth.bf16_bits_to_f32(x[S]).astype(np.float64)
    dl = np.stack([tb[t]["dl"] for t in S]).astype(np.float64)
    err = P.rel_frob(P.to_np(dwr), dl.T @ xf)
    log(f"dW_router [{cfg.E}, {cfg.d}] rel err {err:.3e}")
    assert err <= TOL
    # whole expert gradients of a few used experts
    slots = {}
    for t in S:
        for j in range(cfg.k):
            e = int(idx[t, j])
            if e < cfg.N:
                slots.setdefault(e, []).append((int(t), j))
    multi = [e for e in used if len(slots[e]) > 1]
    check = (multi[:2] + [e for e in used if e not in multi[:2]])[:4]
    for e in check:
        rg = np.zeros((cfg.I, cfg.d))
        ru = np.zeros((cfg.I, cfg.d))
        rd = np.zeros((cfg.d, cfg.I))
        for t, j in slots[e]:
            xt = synth.bf16_bits_to_f32(x[t]).astype(np.float64)
            rg += np.outer(tb[t]["dg"][j], xt)
            ru += np.outer(tb[t]["du"][j], xt)
            rd += np.outer(float(gate[t, j]) * dout[t].astype(np.float64), tb[t]["h"][j])
        for name, g, r in (("dW_gate", dwg, rg), ("dW_up", dwu, ru), ("dW_down", dwd, rd)):
            err = P.rel_frob(P.to_np(g[e]), r)
            log(f"expert {e} ({len(slots[e])} sampled slots) {name} rel err {err:.3e}")
            assert err <= TOL, (e, name, err)
    unused = torch.ones(cfg.N, dtype=torch.bool, device=DEV)
    unused[torch.tensor(used, device=DEV)] = False
    for name, g in (("dW_gate", dwg), ("dW_up", dwu), ("dW_down", dwd)):
        hi, lo = g.amax(dim=(1, 2)), g.amin(dim=(1, 2))  # per expert, no full-size temporaries
        assert float(hi[unused].max()) == 0.0 and float(lo[unused].min()) == 0.0, \
            f"{name} of an expert with no gradient"
    log(f"{int(unused.sum())} experts without a sampled token have zero weight gradients")
    del dinp, dwg, dwu, dwd
    torch.cuda.empty_cache()
