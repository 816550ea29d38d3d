"""HIP-graph capture of the forward and the backward.  The library allocates,
frees and synchronises nothing and records no memset node, so a call can be
captured by a caller that preallocates its buffers (serving loops with few
tokens are launch-bound).  Each captured call is replayed several times,
with eager work (clearing the outputs) and synchronisations between the
replays, and every replay must give bit for bit the eager call's outputs."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("zero_computation_expert_amd")

DEV = "cuda:0"
REPLAYS = 3


def capture(fn):
    """Warm up on a side stream, then capture fn into a graph."""
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("wl", ["tiny", "small"])
def test_forward_graph_replays_match_eager(wl):
    cfg = synth.CONFIGS[wl]
    check_forward_graph(cfg, synth.device_inputs(cfg, DEV))


def test_forward_graph_replays_match_eager_widths_not_multiples_of_8():
    """The zero-padded path (its copy kernels are captured with the rest)."""
    cfg = synth.Config("odd_graph", T=77, d=100, I=36, N=6, Z=3, k=3, dtype="bf16", seed=16)
    h = synth.host_inputs(cfg)
    inp = {n: (torch.from_numpy(v).view(torch.bfloat16) if v.dtype == np.uint16
               else torch.from_numpy(v)).to(DEV) for n, v in h.items()}
    check_forward_graph(cfg, inp)


def check_forward_graph(cfg, inp):
    wl = cfg.name
    args = (inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
            cfg.N, cfg.Z, cfg.k)
    T, E, k = cfg.T, cfg.E, cfg.k
    dt = moe.F32 if cfg.dtype == "f32" else moe.BF16
    ws = torch.empty(max(moe.workspace_bytes(T, cfg.d, cfg.I, cfg.N, cfg.Z, k, dt), 1),
                     dtype=torch.uint8, device=DEV)
    bufs = {"out": torch.empty_like(inp["x"]),
            "counts": torch.empty(E, dtype=torch.int32, device=DEV),
            "topk_idx": torch.empty((T, k), dtype=torch.int32, device=DEV),
            "topk_gate": torch.empty((T, k), dtype=torch.float32, device=DEV)}
    ref = [t.clone() for t in moe.forward(*args)]
    torch.cuda.synchronize()

    g = capture(lambda: moe.forward(*args, workspace=ws, **bufs))
    for rep in range(REPLAYS):
        for t in bufs.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(bufs, bufs.values(), ref):
            assert torch.equal(got, want), (wl, rep, name)
    print(f"[graph] forward {wl}: {REPLAYS} replays equal the eager call", flush=True)


def test_backward_graph_replays_match_eager():
    cfg = synth.Config("graph_bwd", T=300, d=256, I=128, N=8, Z=4, k=3, dtype="bf16", seed=71,
                       bias_lo=-0.01, bias_hi=0.01)
    inp = synth.device_inputs(cfg, DEV)
    _, _, idx, gate = moe.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"],
                                  inp["W_up"], inp["W_down"], cfg.N, cfg.Z, cfg.k)
    dout = synth.device_dout(cfg, DEV)
    args = (inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"], idx, gate, dout,
            cfg.N, cfg.Z)
    ws = torch.empty(moe.backward_workspace_bytes(cfg.T, cfg.d, cfg.I, cfg.N, cfg.Z, cfg.k),
                     dtype=torch.uint8, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    grads = {"dW_router": torch.zeros(cfg.E, cfg.d, **f32),
             "dW_gate": torch.zeros(cfg.N, cfg.I, cfg.d, **f32),
             "dW_up": torch.zeros(cfg.N, cfg.I, cfg.d, **f32),
             "dW_down": torch.zeros(cfg.N, cfg.d, cfg.I, **f32)}
    dx = torch.empty_like(inp["x"])
    ref = [t.clone() for t in moe.backward(*args)]  # weight gradients start from zero
    torch.cuda.synchronize()

    g = capture(lambda: moe.backward(*args, dx=dx, workspace=ws, **grads))
    for rep in range(REPLAYS):
        dx.zero_()
        for t in grads.values():
            t.zero_()  # the weight gradients accumulate: start every replay from zero
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [dx] + list(grads.values())
        for name, a, b in zip(["dx"] + list(grads), got, ref):
            assert torch.equal(a, b), (rep, name)
    print(f"[graph] backward: {REPLAYS} replays equal the eager call", flush=True)
