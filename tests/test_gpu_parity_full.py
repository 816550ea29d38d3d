"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one moe_zc_forward call per workload).

Inputs are generated on the device by the seeded generator; the host copies
the oracle reads (x, W_router, bias) are regenerated on the host and checked
bit-identical to the device ones, and so is one expert per weight tensor.
Routing (index sets, gates, counts) is checked for EVERY token against the
oracle.  Outputs: every token of the small and decode workloads; for prod
and skewed, a cover of every 32-row block of every expert's permuted rows,
so every tile of both expert GEMMs (every expert, row block, chunk and
32-token block, each expert's partial last chunk included) has outputs
compared.  Expert matrices for the oracle are copied from the generator's
device tensors, a few experts at a time (tests/_fullsize.py).
"""
import time

import numpy as np
import pytest

import oracle
import synth
from tests import _fullsize as F
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


def fetch_bf16(dinp):
    return lambda e: tuple(_np16(dinp["W_" + w][e]) for w in ("gate", "up", "down"))


def run_full(cfg, rows_mode):
    t0 = time.time()
    log = lambda m: print(f"[full] {cfg.name}: {m} ({time.time() - t0:.0f}s)", flush=True)  # noqa: E731
    log(f"T={cfg.T} d={cfg.d} I={cfg.I} N={cfg.N} Z={cfg.Z} k={cfg.k}")
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
    log(f"routing ok, near_ties={info['near_ties']} gate_err={info['gate_err']:.2e} "
        f"ffn/token={(idx < cfg.N).sum() / cfg.T:.3f} empty_ffn={(cnt[:cfg.N] == 0).sum()}")

    if rows_mode == "all":
        rows, nblocks = np.arange(cfg.T), None
    else:
        near = np.nonzero(omargin < P.MARGIN)[0][:8]
        rows, nblocks = F.block_cover_rows(idx, cfg.N, extra=list(near) + [0, cfg.T - 1])
    log(f"{len(rows)} tokens to compare" +
        (f" (cover of {nblocks} 32-row blocks)" if nblocks else " (all)"))
    # gates: the oracle's probabilities of the experts the GPU chose (equal to
    # the oracle's own routing outside near-ties)
    g = np.take_along_axis(oprobs, idx.astype(np.int64), 1).astype(np.float32)
    ref = F.streamed_reference(x, cfg.dtype, cfg.N, idx, g, rows, fetch_bf16(dinp), log=log)
    got = P.out_as_f32(out[rows], cfg.dtype)
    assert np.isfinite(P.out_as_f32(out, cfg.dtype)).all()
    err, worst = P.check_outputs(got, ref, cfg.dtype)
    log(f"{len(rows)} tokens rel_frob={err:.3e} worst_token={worst:.3e}")
    return cnt, idx, rows


def test_small_full_size():
    run_full(synth.SMALL, "all")


def test_decode_full_size():
    cnt, idx, _ = run_full(synth.DECODE, "all")
    assert (cnt[: synth.DECODE.N] == 0).any()  # the decode shape leaves experts empty


def test_prod_full_size():
    cnt, idx, rows = run_full(synth.PROD, "cover")
    # every expert above 160 rows (one hot-expert chunk of 256 rows each) has
    # its rows past 160 covered (by construction of the cover; checked here)
    tt, _, ee, pos = F.permuted_positions(idx, synth.PROD.N)
    sel = np.isin(tt, rows)
    for e in np.nonzero(cnt[: synth.PROD.N] > 160)[0]:
        assert (pos[sel & (ee == e)] >= 160).any()


def test_skewed_full_size():
    cnt, idx, rows = run_full(synth.SKEWED, "cover")
    assert cnt[0] == synth.SKEWED.T  # the Zipf head expert takes every token
    # its 64 hot-expert chunks of 256 rows: every 32-row block compared
    tt, _, ee, pos = F.permuted_positions(idx, synth.SKEWED.N)
    hot = np.unique(pos[(ee == 0) & np.isin(tt, rows)] // 32)
    assert hot.size == (synth.SKEWED.T + 31) // 32
    _cache.clear()
    torch.cuda.empty_cache()
