"""GPU parity of the block-scaled FP8 expert path against the oracle.

Quantization (moe_zc_quantize_fp8) is compared byte for byte with the
oracle's.  The forward (moe_zc_forward_fp8) runs on weights that the oracle
quantized on the host, so no oracle input comes from the HIP path; routing
is checked as in the bf16 path (near-tie rule) and outputs against the
oracle recomputed with the GPU's routing, with the bf16 path's tolerances.
At full size (every token at decode; at prod and on the skewed workload a set
of tokens that covers every 32-row block of every expert's rows) the compared tokens' experts are
quantized on the host by the oracle, while the GPU forward uses the GPU
quantizer's output (bit-identical, by the first test)."""
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


def same_bytes(a, b):
    """E4M3 bytes equal, +0 and -0 counted equal."""
    a, b = np.asarray(a, np.uint8), np.asarray(b, np.uint8)
    return (a == b) | (((a & 0x7F) == 0) & ((b & 0x7F) == 0))


def exps_match(e, s):
    return np.array_equal(np.ldexp(1.0, e.astype(np.int64) - 127).astype(np.float32), s)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("block_rows", [128, 1])
def test_quantize_bit_exact(dt, block_rows):
    rng = np.random.default_rng(block_rows + (dt == "f32"))
    shape = (3, 256, 384) if block_rows == 128 else (1, 77, 640)
    w = rng.standard_normal(shape).astype(np.float32)
    w *= rng.choice([1e-30, 1e-3, 1.0, 5e3], size=(shape[0], shape[1], 1)).astype(np.float32)
    w[0, :, :128] = 0.0  # zero blocks
    host = synth.f32_to_bf16_bits(w) if dt == "bf16" else w
    oq, os_ = oracle.quantize_fp8(host, dt, block_rows)
    t = torch.from_numpy(host.view(np.int16) if dt == "bf16" else host)
    t = t.view(torch.bfloat16) if dt == "bf16" else t
    q, e = moe.quantize_fp8(t.to(DEV), block_rows)
    torch.cuda.synchronize()
    assert same_bytes(q.cpu().numpy(), oq).all()
    assert exps_match(e.cpu().numpy(), os_)


def fp8_weights_host(inp):
    return [a for w in ("W_gate", "W_up", "W_down") for a in oracle.quantize_fp8(inp[w], "bf16", 128)]


def run_fp8(cfg, inp, qw, bias=None, scale=1.0):
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(DEV)
    tu8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    # exponent bytes of the oracle's power-of-two scales
    ex = lambda s: tu8((np.frexp(s)[1] - 1 + 127).astype(np.uint8))
    b = torch.from_numpy(np.ascontiguousarray(inp["bias"] if bias is None else bias)).to(DEV)
    qg, sg, qu, su, qd, sd = qw
    out, cnt, idx, gate = moe.forward_fp8(t16(inp["x"]), t16(inp["W_router"]), b, tu8(qg), ex(sg),
                                          tu8(qu), ex(su), tu8(qd), ex(sd), cfg.N, cfg.Z, cfg.k,
                                          routed_scale=scale)
    torch.cuda.synchronize()
    return P.to_np(out), P.to_np(cnt), P.to_np(idx), P.to_np(gate)


def check_fp8(cfg, inp, bias=None, scale=1.0):
    print(f"[fp8] {cfg} routed_scale={scale}", flush=True)
    b = inp["bias"] if bias is None else bias
    qw = fp8_weights_host(inp)
    out, cnt, idx, gate = run_fp8(cfg, inp, qw, bias=b, scale=scale)
    logits = oracle.router_logits(inp["x"], inp["W_router"], "bf16")
    oidx, _, omargin, oprobs = oracle.route_from_logits(logits, b, cfg.k)
    info = P.check_routing(cfg, b, idx, gate, cnt, oidx, oprobs, omargin, scale=scale)
    P.check_counts_against_oracle(cfg, idx, cnt, oidx, omargin)
    g = (np.float32(scale) * np.take_along_axis(oprobs, idx.astype(np.int64), 1)).astype(np.float32)
    ref = oracle.combine_given_routing_fp8(inp["x"], "bf16", cfg.N, idx, g, *qw)
    got = P.out_as_f32(out, "bf16")
    err, worst = P.check_outputs(got, ref, "bf16")
    print(f"[fp8] rel_frob={err:.3e} worst_token={worst:.3e} near_ties={info['near_ties']}",
          flush=True)
    return cnt, idx


FP8_CASES = [
    synth.Config("fp8_ragged", T=300, d=256, I=256, N=10, Z=5, k=4, dtype="bf16", seed=3),
    synth.Config("fp8_wide", T=520, d=384, I=384, N=40, Z=20, k=8, dtype="bf16", seed=5,
                 bias_lo=-0.02, bias_hi=0.02),
    synth.Config("fp8_decodeish", T=9, d=512, I=256, N=48, Z=16, k=6, dtype="bf16", seed=6),
]


@pytest.mark.parametrize("cfg", FP8_CASES, ids=lambda c: c.name)
def test_fp8_forward_parity(cfg):
    check_fp8(cfg, synth.host_inputs(cfg))


def test_fp8_routed_scale():
    check_fp8(FP8_CASES[0], synth.host_inputs(FP8_CASES[0]), scale=1.75)


def test_fp8_hot_expert_spans_many_chunks():
    cfg = synth.Config("fp8_hot", T=700, d=256, I=128, N=12, Z=4, k=3, dtype="bf16", seed=11)
    inp = synth.host_inputs(cfg)
    b = inp["bias"].copy()
    b[3] = 10.0
    cnt, idx = check_fp8(cfg, inp, bias=b)
    assert cnt[3] == cfg.T


def test_fp8_all_zero_routing_reads_no_expert_weights():
    cfg = synth.Config("fp8_zero", T=130, d=128, I=128, N=6, Z=5, k=4, dtype="bf16", seed=8)
    inp = synth.host_inputs(cfg)
    b = np.zeros(cfg.E, np.float32)
    b[cfg.N:] = 10.0
    qw = [np.full_like(a, 0x7F) if a.dtype == np.uint8 else a for a in fp8_weights_host(inp)]
    out, cnt, idx, gate = run_fp8(cfg, inp, qw, bias=b)  # E4M3 NaN bytes in every expert
    assert (idx >= cfg.N).all()
    ref = gate.astype(np.float64).sum(1)[:, None] * P.out_as_f32(inp["x"], "bf16")
    got = P.out_as_f32(out, "bf16")
    assert np.isfinite(got).all() and P.rel_frob(got, ref) <= 2e-2


def run_fp8_full_cover(cfg, tag):
    """Full-size FP8 forward: routing on every token, and the output of a
    cover of every 32-row block of every expert's permuted rows (every tile
    of both FP8 expert GEMMs, each expert's partial last chunk included)
    against the FP8 oracle.  The GPU forward runs on the GPU quantizer's
    weights (bit-identical to the oracle's, first test); the oracle
    quantizes each routed expert's bf16 matrices itself, on the host,
    streaming a few experts at a time."""
    t0 = time.time()
    log = lambda m: print(f"[fp8 {tag}] {m} ({time.time() - t0:.0f}s)", flush=True)  # noqa: E731
    dinp = synth.device_inputs(cfg, DEV)
    qg, eg = moe.quantize_fp8(dinp["W_gate"], 128)
    qu, eu = moe.quantize_fp8(dinp["W_up"], 128)
    qd, ed = moe.quantize_fp8(dinp["W_down"], 128)
    out, cnt, idx, gate = moe.forward_fp8(dinp["x"], dinp["W_router"], dinp["bias"], qg, eg, qu, eu,
                                          qd, ed, cfg.N, cfg.Z, cfg.k)
    torch.cuda.synchronize()
    del qg, qu, qd, eg, eu, ed
    torch.cuda.empty_cache()
    out, cnt, idx, gate = P.to_np(out), P.to_np(cnt), P.to_np(idx), P.to_np(gate)
    x, wr, bias = synth.host_x(cfg), synth.host_router(cfg), synth.host_bias(cfg)
    assert (x == P.to_np(dinp["x"])).all()
    logits = oracle.router_logits(x, wr, "bf16")
    oidx, _, omargin, oprobs = oracle.route_from_logits(logits, bias, cfg.k)
    info = P.check_routing(cfg, bias, idx, gate, cnt, oidx, oprobs, omargin)
    P.check_counts_against_oracle(cfg, idx, cnt, oidx, omargin)
    near = np.nonzero(omargin < P.MARGIN)[0][:8]
    rows, nblocks = F.block_cover_rows(idx, cfg.N, extra=list(near) + [0, cfg.T - 1])
    log(f"routing ok, near_ties={info['near_ties']}; {len(rows)} tokens cover {nblocks} blocks, "
        f"largest expert {int(cnt[: cfg.N].max())} rows")

    def fetch(e):
        mats = [P.to_np(dinp["W_" + w][e]) for w in ("gate", "up", "down")]
        return tuple(a for m in mats for a in oracle.quantize_fp8(m, "bf16", 128))

    g = np.take_along_axis(oprobs, idx.astype(np.int64), 1).astype(np.float32)
    ref = F.streamed_reference(x, "bf16", cfg.N, idx, g, rows, fetch, ffn=oracle.ffn_pairs_fp8,
                               log=log)
    assert np.isfinite(P.out_as_f32(out, "bf16")).all()
    err, worst = P.check_outputs(P.out_as_f32(out[rows], "bf16"), ref, "bf16")
    log(f"{len(rows)} tokens rel_frob={err:.3e} worst_token={worst:.3e}")
    del dinp
    torch.cuda.empty_cache()


def test_fp8_prod_full_size_block_cover():
    """Production shapes (T=8192, d=6144, 512 SwiGLU experts of 2048, 256 zero
    experts, top-12) with FP8 experts."""
    run_fp8_full_cover(synth.PROD, "prod")


def test_fp8_skewed_full_size_block_cover():
    """The skewed workload (T=16384, one expert chosen by every token) with
    FP8 experts: the hot expert's 103 chunks of 160 rows, in groups of 8 per
    row block, every 32-row block compared."""
    run_fp8_full_cover(synth.SKEWED, "skewed")


def test_fp8_decode_full_size_every_token():
    """The decode shape (T=128, d=6144, 512 SwiGLU experts of 2048, 256 zero
    experts, top-12) with FP8 experts: routing on every token, and the
    output of every token against the FP8 oracle.  The GPU forward runs on
    the GPU quantizer's weights (bit-identical to the oracle's, first test);
    the oracle quantizes each routed expert's bf16 matrices itself, on the
    host, streaming a few experts at a time."""
    cfg = synth.DECODE
    t0 = time.time()
    log = lambda m: print(f"[fp8 decode] {m} ({time.time() - t0:.0f}s)", flush=True)  # noqa: E731
    big = cfg.with_(T=cfg.T)
    dinp = synth.device_inputs(big, DEV)
    qg, eg = moe.quantize_fp8(dinp["W_gate"], 128)
    qu, eu = moe.quantize_fp8(dinp["W_up"], 128)
    qd, ed = moe.quantize_fp8(dinp["W_down"], 128)
    out, cnt, idx, gate = moe.forward_fp8(dinp["x"], dinp["W_router"], dinp["bias"], qg, eg, qu, eu,
                                          qd, ed, cfg.N, cfg.Z, cfg.k)
    torch.cuda.synchronize()
    del qg, qu, qd, eg, eu, ed
    out, cnt, idx, gate = P.to_np(out), P.to_np(cnt), P.to_np(idx), P.to_np(gate)
    x, wr, bias = synth.host_x(cfg), synth.host_router(cfg), synth.host_bias(cfg)
    assert (x == P.to_np(dinp["x"])).all()
    logits = oracle.router_logits(x, wr, "bf16")
    oidx, _, omargin, oprobs = oracle.route_from_logits(logits, bias, cfg.k)
    info = P.check_routing(cfg, bias, idx, gate, cnt, oidx, oprobs, omargin)
    P.check_counts_against_oracle(cfg, idx, cnt, oidx, omargin)
    log(f"routing ok, near_ties={info['near_ties']}, {int((cnt[:cfg.N] > 0).sum())} experts used")

    def fetch(e):
        mats = [P.to_np(dinp["W_" + w][e]) for w in ("gate", "up", "down")]
        return tuple(a for m in mats for a in oracle.quantize_fp8(m, "bf16", 128))

    g = np.take_along_axis(oprobs, idx.astype(np.int64), 1).astype(np.float32)
    ref = F.streamed_reference(x, "bf16", cfg.N, idx, g, np.arange(cfg.T), fetch,
                               ffn=oracle.ffn_pairs_fp8, log=log)
    err, worst = P.check_outputs(P.out_as_f32(out, "bf16"), ref, "bf16")
    log(f"all {cfg.T} tokens rel_frob={err:.3e} worst_token={worst:.3e}")
    del dinp
    torch.cuda.empty_cache()
