"""GPU checks of the dense SwiGLU FFN (moe_zc_dense_ffn) and of the
two-stream ScMoE schedule (moe_zc_scmoe_forward), through the C ABI.

The dense FFN is compared with the oracle's (2e-2 relative Frobenius, every
token within 1.5x).  The schedule is compared with itself: the MoE chunks on
one stream and the dense FFN on another must give bit for bit what the same
calls give on a single stream, and the chunked MoE output is checked against
the oracle as the forward's parity tests do."""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("zero_computation_expert_amd")

DEV = "cuda:0"


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(DEV)


def bf16_np(t):
    return synth.bf16_bits_to_f32(P.to_np(t))


@pytest.mark.parametrize("T,d,Id", [(300, 256, 640), (37, 128, 96), (1, 64, 64), (170, 200, 72)])
def test_dense_ffn_parity(T, d, Id):
    cfg = synth.Config("dense", T=T, d=d, I=64, N=1, Z=1, k=1, dtype="bf16", seed=62)
    w = synth.host_dense(cfg, Id)
    out = moe.dense_ffn(dev_bf16(w["x_dense"]), dev_bf16(w["W1"]), dev_bf16(w["W3"]),
                        dev_bf16(w["W2"]))
    torch.cuda.synchronize()
    ref = oracle.dense_ffn(w["x_dense"], w["W1"], w["W3"], w["W2"], "bf16")
    err, worst = P.check_outputs(bf16_np(out), ref, "bf16")
    print(f"[dense] T={T} d={d} I={Id} rel_frob={err:.3e} worst_token={worst:.3e}", flush=True)


def test_dense_ffn_production_width_sampled():
    """The production shape of the dense path: T=8192, d=6144, width 12288;
    sampled tokens against the oracle (weights copied from the device
    generator's own tensors)."""
    cfg = synth.PROD
    w = synth.device_dense(cfg, synth.DENSE_WIDTH)
    out = moe.dense_ffn(w["x_dense"], w["W1"], w["W3"], w["W2"])
    torch.cuda.synchronize()
    toks = [0, 1, 4095, 5000, cfg.T - 1]
    host = {k: P.to_np(v) for k, v in w.items() if k != "x_dense"}
    x = P.to_np(w["x_dense"][toks])
    ref = oracle.dense_ffn(x, host["W1"], host["W3"], host["W2"], "bf16")
    err, worst = P.check_outputs(bf16_np(out[toks]), ref, "bf16")
    print(f"[dense prod] rel_frob={err:.3e} worst_token={worst:.3e}", flush=True)


def _scmoe_inputs(cfg, Id):
    return synth.device_inputs(cfg, DEV), synth.device_dense(cfg, Id, DEV)


def _run(cfg, inp, dn, nchunks, two_streams):
    s0 = torch.cuda.current_stream(DEV)
    s1 = torch.cuda.Stream(device=DEV) if two_streams else s0
    s1.wait_stream(s0)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    om, od, cnt, idx, gate = moe.scmoe_forward(
        inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
        dn["x_dense"], dn["W1"], dn["W3"], dn["W2"], cfg.N, cfg.Z, cfg.k, nchunks, s0, s1,
        topk_idx=idx, topk_gate=gate)
    s0.wait_stream(s1)
    torch.cuda.synchronize()
    return {"out_moe": P.to_np(om), "out_dense": P.to_np(od), "counts": P.to_np(cnt),
            "idx": P.to_np(idx), "gate": P.to_np(gate)}


@pytest.mark.parametrize("nchunks", [1, 2])
def test_scmoe_two_streams_equal_one_stream(nchunks):
    cfg = synth.Config("scmoe", T=300, d=256, I=128, N=8, Z=4, k=3, dtype="bf16", seed=63,
                       bias_lo=-0.01, bias_hi=0.01)
    inp, dn = _scmoe_inputs(cfg, 512)
    a = _run(cfg, inp, dn, nchunks, False)
    b = _run(cfg, inp, dn, nchunks, True)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    assert a["counts"].shape == (nchunks, cfg.E)
    assert (a["counts"].sum(0) == np.bincount(a["idx"].ravel(), minlength=cfg.E)).all()
    # the dense output is the dense FFN's, the MoE output the forward's
    h = synth.host_dense(cfg, 512)
    ref = oracle.dense_ffn(h["x_dense"], h["W1"], h["W3"], h["W2"], "bf16")
    P.check_outputs(synth.bf16_bits_to_f32(a["out_dense"]), ref, "bf16")
    hin = synth.host_inputs(cfg)
    logits = oracle.router_logits(hin["x"], hin["W_router"], "bf16")
    oidx, _, omargin, oprobs = oracle.route_from_logits(logits, hin["bias"], cfg.k)
    P.check_routing(cfg, hin["bias"], a["idx"], a["gate"], a["counts"].sum(0), oidx, oprobs,
                    omargin)
    mref = P.reference_outputs(cfg, hin, a["idx"], oprobs)
    err, worst = P.check_outputs(synth.bf16_bits_to_f32(a["out_moe"]), mref, "bf16")
    print(f"[scmoe] nchunks={nchunks} moe rel_frob={err:.3e}", flush=True)


def test_scmoe_production_shape_two_streams_equal_one_stream():
    cfg = synth.PROD
    inp, dn = _scmoe_inputs(cfg, synth.DENSE_WIDTH)
    a = _run(cfg, inp, dn, 2, False)
    b = _run(cfg, inp, dn, 2, True)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    assert a["counts"].sum() == cfg.T * cfg.k
