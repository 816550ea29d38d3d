"""GPU parity of the bias controller (moe_zc_bias_update) against the
oracle: bit-exact (fp32 elementwise, same operation order, no contraction),
alone and in a closed loop with the GPU forward."""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("zero_computation_expert_amd")
DEV = "cuda:0"


@pytest.mark.parametrize("E", [1, 5, 300, 768, 2048, 4099])
@pytest.mark.parametrize("mode,with_state", [(0, True), (0, False), (1, False)])
def test_bias_update_bit_exact(E, mode, with_state):
    rng = np.random.default_rng(E * 7 + mode * 3 + with_state)
    T = int(rng.integers(1, 20000))
    counts = rng.integers(0, 3 * T, E).astype(np.int32)
    target = (rng.random(E) * 3 * T).astype(np.float32)
    target[: E // 3] = counts[: E // 3]  # some experts exactly on target
    bias = rng.normal(0, 1e-2, E).astype(np.float32)
    state = rng.normal(0, 1e-1, 2 * E).astype(np.float32) if with_state else None
    lr, ki, kp, kd = (float(np.float32(v)) for v in rng.random(4) * [1e-2, 1.5, 0.8, 0.3])
    ob, ost = oracle.bias_update(counts, target, bias, T, lr, ki, kp, kd, state, mode)
    gb = torch.from_numpy(bias.copy()).to(DEV)
    gst = torch.from_numpy(state.copy()).to(DEV) if with_state else None
    moe.bias_update(torch.from_numpy(counts).to(DEV), torch.from_numpy(target).to(DEV), gb, T,
                    lr, ki, kp, kd, gst, mode)
    torch.cuda.synchronize()
    assert (gb.cpu().numpy().view(np.uint32) == ob.view(np.uint32)).all()
    if with_state:
        assert (gst.cpu().numpy().view(np.uint32) == ost.view(np.uint32)).all()


def test_closed_loop_with_the_gpu_forward():
    """Forward + controller on the GPU, repeated on one batch, against the
    oracle doing the same.  Each iteration: the GPU routing is checked
    against the oracle's under the near-tie rule, both controllers are fed
    the GPU's counts and must produce bit-identical biases (so both sides
    route with the same bias next time), and the FFN share reaches its
    target."""
    cfg = synth.Config("loop", T=512, d=64, I=16, N=8, Z=8, k=4, dtype="f32", seed=21,
                       bias_lo=0.0, bias_hi=0.0)
    inp = synth.host_inputs(cfg)
    E, T, k, N = cfg.E, cfg.T, cfg.k, cfg.N
    target = np.empty(E, np.float32)
    target[:N] = 0.75 * T * k / N
    target[N:] = 0.25 * T * k / cfg.Z
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    x, wr, wg, wu, wd = (t(inp[n]) for n in ("x", "W_router", "W_gate", "W_up", "W_down"))
    gbias, gstate, gtarget = t(np.zeros(E, np.float32)), t(np.zeros(2 * E, np.float32)), t(target)
    obias, ostate = np.zeros(E, np.float32), np.zeros(2 * E, np.float32)
    logits = oracle.router_logits(inp["x"], inp["W_router"], "f32")
    near = 0
    for it in range(120):
        lr = float(np.float32(0.02 * 0.99 ** it))
        _, gcnt, gidx, _ = moe.forward(x, wr, gbias, wg, wu, wd, N, cfg.Z, k)
        moe.bias_update(gcnt, gtarget, gbias, T, lr, 1.0, 0.5, 0.0, gstate, 0)
        oidx, _, omargin, _ = oracle.route_from_logits(logits, obias, k)
        torch.cuda.synchronize()
        cnt = gcnt.cpu().numpy()
        P.check_counts_against_oracle(cfg, gidx.cpu().numpy(), cnt, oidx, omargin)
        near += int((omargin < P.MARGIN).sum())
        obias, ostate = oracle.bias_update(cnt, target, obias, T, lr, 1.0, 0.5, 0.0, ostate, 0)
        assert (gbias.cpu().numpy().view(np.uint32) == obias.view(np.uint32)).all(), it
        assert (gstate.cpu().numpy().view(np.uint32) == ostate.view(np.uint32)).all(), it
    print(f"[loop] near-tie token-iterations: {near}", flush=True)
    share = cnt[:N].sum() / (T * k)
    assert abs(share - 0.75) < 0.02
