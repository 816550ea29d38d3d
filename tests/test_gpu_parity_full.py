"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one moe_zc_forward call per workload).

Inputs are generated on the device by the seeded generator; the host copies
the oracle reads (x, W_router, bias) are regenerated on the host and checked
bit-identical to the device ones, and so is one expert per weight tensor.
Routing (index sets, gates, counts) is checked for EVERY token against the
oracle; outputs are checked on sampled tokens (the oracle computes them one
by one), using the sampled tokens' expert matrices copied from the
generator's device tensors.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("zero_computation_expert_amd")

DEV = "cuda:0"
_cache = {}


def _np16(t):
    return P.to_np(t)


def device_weights(cfg):
    """Device inputs; the d=6144 workloads share weights (same seeds and shapes)."""
    key = (cfg.d, cfg.I, cfg.N, cfg.Z, cfg.dtype, cfg.seed)
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        big = cfg.with_(T=max(cfg.T, synth.SKEWED.T if cfg.d == 6144 else cfg.T))
        _cache[key] = synth.device_inputs(big, DEV)
        torch.cuda.synchronize()
    inp = dict(_cache[key])
    inp["x"] = inp["x"][: cfg.T]
    inp["bias"] = torch.from_numpy(synth.host_bias(cfg)).to(DEV)
    return inp


def _sample_rows(cfg, margin, n):
    rng = np.random.default_rng(0)
    rows = set(rng.choice(cfg.T, size=min(n, cfg.T), replace=False).tolist())
    rows |= {0, cfg.T - 1}
    rows |= set(np.nonzero(margin < P.MARGIN)[0][:3].tolist())
    return np.array(sorted(rows))


def run_full(cfg, n_sample):
    print(f"[full] {cfg.name}: T={cfg.T} d={cfg.d} I={cfg.I} N={cfg.N} Z={cfg.Z} k={cfg.k}",
          flush=True)
    dinp = device_weights(cfg)
    out, cnt, idx, gate = moe.forward(dinp["x"], dinp["W_router"], dinp["bias"], dinp["W_gate"],
                                      dinp["W_up"], dinp["W_down"], cfg.N, cfg.Z, cfg.k)
    torch.cuda.synchronize()
    out, cnt, idx, gate = _np16(out), _np16(cnt), _np16(idx), _np16(gate)

    # host copies of what the oracle reads, bit-identical to the device ones
    x = synth.host_x(cfg)
    wr = synth.host_router(cfg)
    bias = synth.host_bias(cfg)
    assert (x == _np16(dinp["x"])).all() and (wr == _np16(dinp["W_router"])).all()
    for w in ("gate", "up", "down"):
        assert (synth.host_expert(cfg, w, cfg.N - 1) == _np16(dinp["W_" + w][cfg.N - 1:])).all()

    logits = oracle.router_logits(x, wr, cfg.dtype)
    oidx, _, omargin, oprobs = oracle.route_from_logits(logits, bias, cfg.k)
    info = P.check_routing(cfg, bias, idx, gate, cnt, oidx, oprobs, omargin)
    P.check_counts_against_oracle(cfg, idx, cnt, oidx, omargin)
    print(f"[full] {cfg.name}: routing ok, near_ties={info['near_ties']} "
          f"gate_err={info['gate_err']:.2e} ffn/token={(idx < cfg.N).sum() / cfg.T:.3f} "
          f"empty_ffn={(cnt[:cfg.N] == 0).sum()}", flush=True)

    rows = _sample_rows(cfg, omargin, n_sample)

    def one(t):
        experts = {}
        for e in idx[t]:
            e = int(e)
            if e < cfg.N:
                experts[e] = tuple(_np16(dinp["W_" + w][e]) for w in ("gate", "up", "down"))
        g = oprobs[t, idx[t]].astype(np.float32)
        return oracle.token_output(x[t], cfg.dtype, cfg.N, idx[t], g, experts)

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        ref = np.stack(list(ex.map(one, rows)))
    got = P.out_as_f32(out[rows], cfg.dtype)
    assert np.isfinite(P.out_as_f32(out, cfg.dtype)).all()
    err, worst = P.check_outputs(got, ref, cfg.dtype)
    print(f"[full] {cfg.name}: sampled {len(rows)} tokens rel_frob={err:.3e} "
          f"worst_token={worst:.3e}", flush=True)
    return cnt, idx


def test_small_full_size():
    run_full(synth.SMALL, 48)


def test_decode_full_size():
    cnt, idx = run_full(synth.DECODE, 24)
    assert (cnt[: synth.DECODE.N] == 0).any()  # the decode shape leaves experts empty


def test_prod_full_size():
    run_full(synth.PROD, 16)


def test_skewed_full_size():
    cnt, _ = run_full(synth.SKEWED, 16)
    assert cnt[0] == synth.SKEWED.T  # the Zipf head expert takes every token
    _cache.clear()
    torch.cuda.empty_cache()
