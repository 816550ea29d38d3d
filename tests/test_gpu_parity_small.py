"""GPU parity against the CPU oracle on shapes the oracle finishes in seconds
(full element-by-element comparison), plus the method's edge cases.  All
calls go through the C ABI (zero_computation_expert_amd.forward)."""
import numpy as np
import pytest

import oracle
import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("zero_computation_expert_amd")


def run_gpu(cfg, inp, bias=None, poison=False, scale=1.0, **over):
    dev = "cuda:0"
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16

    def dt(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        if cfg.dtype == "bf16":
            t = t.view(torch.bfloat16)
        return t.to(dev)

    x = dt(inp["x"])
    b = torch.from_numpy(np.ascontiguousarray(inp["bias"] if bias is None else bias)).to(dev)
    ws = None
    if poison:
        nbytes = moe.workspace_bytes(cfg.T, cfg.d, cfg.I, cfg.N, cfg.Z, cfg.k,
                                     moe.F32 if cfg.dtype == "f32" else moe.BF16)
        ws = torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=dev)  # NaN bytes
    out, cnt, idx, gate = moe.forward(x, dt(inp["W_router"]), b, dt(over.get("W_gate", inp["W_gate"])),
                                      dt(over.get("W_up", inp["W_up"])),
                                      dt(over.get("W_down", inp["W_down"])),
                                      cfg.N, cfg.Z, cfg.k, workspace=ws, routed_scale=scale)
    torch.cuda.synchronize()
    assert out.dtype == tdt
    return P.to_np(out), P.to_np(cnt), P.to_np(idx), P.to_np(gate)


def oracle_routing(cfg, inp, bias=None):
    logits = oracle.router_logits(inp["x"], inp["W_router"], cfg.dtype)
    b = inp["bias"] if bias is None else bias
    return oracle.route_from_logits(logits, b, cfg.k)


def full_check(cfg, inp, bias=None, poison=False, scale=1.0):
    print(f"[parity] {cfg} routed_scale={scale}", flush=True)
    b = inp["bias"] if bias is None else bias
    out, cnt, idx, gate = run_gpu(cfg, inp, bias=b, poison=poison, scale=scale)
    oidx, ogate, omargin, oprobs = oracle_routing(cfg, inp, b)
    info = P.check_routing(cfg, b, idx, gate, cnt, oidx, oprobs, omargin, scale=scale)
    P.check_counts_against_oracle(cfg, idx, cnt, oidx, omargin)
    ref = P.reference_outputs(cfg, inp, idx, oprobs, scale=scale)
    got = P.out_as_f32(out, cfg.dtype)
    err, worst = P.check_outputs(got, ref, cfg.dtype)
    print(f"[parity] rel_frob={err:.3e} worst_token={worst:.3e} gate_err={info['gate_err']:.2e} "
          f"near_ties={info['near_ties']}", flush=True)
    return out, cnt, idx, gate


# tiny config of the workload table (fp32) and ragged shapes that span several
# tiles with partial row blocks, partial token chunks and a K tail
RAGGED = [
    synth.TINY,
    synth.Config("ragged_bf16", T=300, d=256, I=192, N=10, Z=5, k=4, dtype="bf16", seed=3),
    synth.Config("ragged_f32", T=300, d=256, I=192, N=10, Z=5, k=4, dtype="f32", seed=3),
    synth.Config("ktail_bf16", T=77, d=200, I=72, N=5, Z=3, k=3, dtype="bf16", seed=4),
    synth.Config("ktail_f32", T=77, d=200, I=72, N=5, Z=3, k=3, dtype="f32", seed=4),
    synth.Config("wide_bf16", T=520, d=384, I=320, N=40, Z=20, k=8, dtype="bf16", seed=5,
                 bias_lo=-0.02, bias_hi=0.02),
    synth.Config("decodeish_bf16", T=9, d=512, I=256, N=48, Z=16, k=6, dtype="bf16", seed=6),
]


@pytest.mark.parametrize("cfg", RAGGED, ids=lambda c: c.name)
def test_parity_full(cfg):
    full_check(cfg, synth.host_inputs(cfg), poison=True)


# widths that are not multiples of 8: the forward's zero-padded path (one
# element per row up to a whole 16-byte piece short), every element compared
ODD = [
    synth.Config("odd_bf16", T=77, d=100, I=36, N=6, Z=3, k=3, dtype="bf16", seed=16),
    synth.Config("odd_f32", T=77, d=100, I=36, N=6, Z=3, k=3, dtype="f32", seed=16),
    synth.Config("odd_narrow_bf16", T=33, d=13, I=5, N=4, Z=2, k=2, dtype="bf16", seed=17),
    synth.Config("odd_one_bf16", T=20, d=1, I=1, N=3, Z=2, k=2, dtype="bf16", seed=19),
    synth.Config("odd_d_only_bf16", T=300, d=1001, I=256, N=10, Z=5, k=4, dtype="bf16", seed=18),
    synth.Config("odd_I_only_f32", T=170, d=256, I=250, N=12, Z=4, k=4, dtype="f32", seed=20),
]


@pytest.mark.parametrize("cfg", ODD, ids=lambda c: c.name)
def test_widths_not_multiples_of_8(cfg):
    full_check(cfg, synth.host_inputs(cfg), poison=True)


@pytest.mark.parametrize("cfg,scale", [(RAGGED[1], 2.5), (RAGGED[2], 2.5), (RAGGED[5], 0.37)],
                         ids=["bf16-2.5", "f32-2.5", "wide-0.37"])
def test_routed_scale(cfg, scale):
    """Gates = routed_scale * p on every slot: routing identical to the
    unscaled call, gates and outputs against the oracle with the same scale
    (an FFN-only or selection-side scale would fail the output check)."""
    inp = synth.host_inputs(cfg)
    out, cnt, idx, gate = full_check(cfg, inp, poison=True, scale=scale)
    _, cnt1, idx1, gate1 = run_gpu(cfg, inp)
    assert np.array_equal(idx, idx1) and np.array_equal(cnt, cnt1)
    assert np.array_equal(gate, (np.float32(scale) * gate1).astype(np.float32))


def test_routed_scale_all_zero_routing():
    """Every slot on a zero expert: out = (sum of the scaled gates) * x."""
    cfg = synth.Config("allzero_s", T=70, d=128, I=64, N=6, Z=5, k=4, dtype="f32", seed=15)
    inp = synth.host_inputs(cfg)
    b = np.zeros(cfg.E, np.float32)
    b[cfg.N:] = 10.0
    out, cnt, idx, gate = run_gpu(cfg, inp, bias=b, scale=3.0)
    assert (idx >= cfg.N).all()
    ref = gate.astype(np.float64).sum(1)[:, None] * inp["x"].astype(np.float64)
    assert P.rel_frob(out, ref) <= P.OUT_TOL["f32"]
    _, _, _, oprobs = oracle_routing(cfg, inp, b)
    assert np.abs(gate - 3.0 * np.take_along_axis(oprobs, idx.astype(np.int64), 1)).max() <= 3e-5


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_split_router_slices_summed_before_topk(dt):
    """Few tokens, many experts, wide d: the router GEMM splits K into 16
    slices and, with only 8 top-k blocks, the slices are summed by a separate
    kernel before top-k.  T*E is odd here, so that kernel takes its
    one-logit-per-thread form."""
    cfg = synth.Config("split16_" + dt, T=127, d=2048, I=16, N=515, Z=256, k=12, dtype=dt,
                       seed=17, bias_lo=-1e-3, bias_hi=1e-3)
    assert (cfg.T * cfg.E) % 2 == 1
    full_check(cfg, synth.host_inputs(cfg), poison=True)


def test_maximum_expert_count_and_k():
    """The library's limits: E = 2048 experts (1024 FFN + 1024 zero), k = 64
    slots per token; the widest top-k variant and 8 router row blocks."""
    cfg = synth.Config("maxE", T=40, d=64, I=16, N=1024, Z=1024, k=64, dtype="bf16", seed=13,
                       bias_lo=-1e-4, bias_hi=1e-4)
    full_check(cfg, synth.host_inputs(cfg), poison=True)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_exact_ties_go_to_the_lower_index(dt):
    """Every expert gets the same router row, so all probabilities are bit-equal,
    and the bias splits the 200 experts into 32 groups (e mod 32) of equal,
    well separated values.  Selection must take the groups by bias, and within
    a group ascending expert index: ties between lanes of the top-k kernel
    (e, e + 32) and between register slots of one lane (e, e + 64), with k
    reaching into the second group.  The near-tie exclusion of the parity
    tests does not apply here: the expected indices are exact."""
    cfg = synth.Config("ties", T=70, d=128, I=64, N=150, Z=50, k=12, dtype=dt, seed=21)
    inp = synth.host_inputs(cfg)
    inp["W_router"] = np.ascontiguousarray(np.broadcast_to(inp["W_router"][:1], inp["W_router"].shape))
    grp = np.random.default_rng(21).permutation(32).astype(np.float32)
    bias = (grp * np.float32(1e-3))[np.arange(cfg.E) % 32]
    out, cnt, idx, gate = run_gpu(cfg, inp, bias=bias)
    want = sorted(range(cfg.E), key=lambda e: (-float(bias[e]), e))[: cfg.k]
    assert want[0] % 32 == want[6] % 32 != want[7] % 32  # 7 in the top group, then the next
    assert (idx == np.array(want, np.int32)[None, :]).all()
    assert (gate == gate[0, 0]).all() and abs(float(gate[0, 0]) - 1.0 / cfg.E) < 1e-6
    expect_cnt = np.zeros(cfg.E, np.int64)
    expect_cnt[want] = cfg.T
    assert (cnt == expect_cnt).all()
    _, _, _, oprobs = oracle_routing(cfg, inp, bias)
    ref = P.reference_outputs(cfg, inp, idx, oprobs)
    err, _ = P.check_outputs(P.out_as_f32(out, dt), ref, dt)
    print(f"[ties] {dt}: selection exact, rel_frob={err:.3e}", flush=True)


def test_routing_and_outputs_fuzz():
    """40 seeded random shapes across the top-k kernel's register layouts (1 to
    2048 experts: 1 to 32 scores per lane, lanes with no expert, N or Z zero),
    k from 1 to min(64, E) (k = E included), a bias that dominates the
    probabilities, none, or one of their size, both dtypes: routing and counts
    against the oracle (near-tie rule), outputs where FFN experts exist."""
    rng = np.random.default_rng(1234)
    seen_k_eq_e = False
    for i in range(40):
        E = int(rng.choice([1, 2, 7, 63, 64, 65, 100, 255, 256, 257, 768, 1000, 2048]))
        N = int(rng.integers(0, E + 1))
        k = int(rng.integers(1, min(64, E) + 1)) if i % 8 else min(64, E)
        seen_k_eq_e |= k == E
        scale = float(rng.choice([0.0, 1e-4, 0.1]))
        cfg = synth.Config(f"fuzz{i}", T=int(rng.integers(1, 150)), d=int(rng.choice([8, 64, 136])),
                           I=8, N=N, Z=E - N, k=k, dtype=str(rng.choice(["bf16", "f32"])),
                           seed=100 + i, bias_lo=-scale, bias_hi=scale)
        print(f"[fuzz] {cfg}", flush=True)
        inp = synth.host_inputs(cfg)
        out, cnt, idx, gate = run_gpu(cfg, inp)
        oidx, _, omargin, oprobs = oracle_routing(cfg, inp)
        P.check_routing(cfg, inp["bias"], idx, gate, cnt, oidx, oprobs, omargin)
        P.check_counts_against_oracle(cfg, idx, cnt, oidx, omargin)
        if N > 0:
            ref = P.reference_outputs(cfg, inp, idx, oprobs)
            P.check_outputs(P.out_as_f32(out, cfg.dtype), ref, cfg.dtype)
    assert seen_k_eq_e


@pytest.mark.parametrize("k", [4, 5, 8, 9, 12, 13, 16, 17, 33])
def test_combine_every_batch_size(k):
    """The combine loads each token's slots in batches whose size it picks
    from k (4, 8, 12 or 16): every size, one slot past it, and several
    batches (k = 33), bf16 and all elements against the oracle."""
    cfg = synth.Config(f"k{k}", T=40, d=128, I=64, N=24, Z=16, k=k, dtype="bf16", seed=200 + k)
    full_check(cfg, synth.host_inputs(cfg), poison=True)


def test_deterministic_bitwise():
    cfg = RAGGED[1]
    inp = synth.host_inputs(cfg)
    a = run_gpu(cfg, inp)
    b = run_gpu(cfg, inp, poison=True)
    for u, v in zip(a, b):
        assert (u == v).all()


def test_token_permutation_equivariance():
    cfg = RAGGED[1]
    inp = synth.host_inputs(cfg)
    a = run_gpu(cfg, inp)
    perm = np.random.default_rng(0).permutation(cfg.T)
    inp2 = dict(inp, x=inp["x"][perm])
    b = run_gpu(cfg, inp2)
    assert (b[2] == a[2][perm]).all() and (b[1] == a[1]).all()
    assert P.rel_frob(P.out_as_f32(b[0], cfg.dtype), P.out_as_f32(a[0], cfg.dtype)[perm]) < 1e-6


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_all_zero_routing_is_gate_sum_times_x(dt):
    """Bias +10 on every zero expert (Z >= k): no FFN expert runs, out = (sum of
    gates) * x.  The FFN weights are NaN: reading them would show."""
    cfg = synth.Config("allzero", T=130, d=128, I=64, N=6, Z=5, k=4, dtype=dt, seed=8)
    inp = synth.host_inputs(cfg)
    b = np.zeros(cfg.E, np.float32)
    b[cfg.N:] = 10.0
    nan = np.full_like(inp["W_gate"], 0x7FC0 if dt == "bf16" else np.float32("nan"))
    inp_nan = dict(inp, W_gate=nan, W_up=nan, W_down=nan.copy())
    out, cnt, idx, gate = run_gpu(cfg, inp_nan, bias=b)
    assert (idx >= cfg.N).all() and (cnt[:cfg.N] == 0).all()
    x = P.out_as_f32(inp["x"], dt)
    zs = gate.astype(np.float64).sum(1)
    ref = zs[:, None] * x
    assert P.rel_frob(P.out_as_f32(out, dt), ref) <= P.OUT_TOL[dt]
    assert np.isfinite(P.out_as_f32(out, dt)).all()


def test_no_ffn_experts():
    cfg = synth.Config("n0", T=70, d=64, I=8, N=0, Z=6, k=3, dtype="bf16", seed=2)
    x, wr, bias = synth.host_x(cfg), synth.host_router(cfg), synth.host_bias(cfg)
    inp = {"x": x, "W_router": wr, "bias": bias, "W_gate": None, "W_up": None, "W_down": None}
    out, cnt, idx, gate = run_gpu(cfg, inp)
    oidx, ogate, omargin, oprobs = oracle_routing(cfg, inp)
    P.check_routing(cfg, bias, idx, gate, cnt, oidx, oprobs, omargin)
    ref = gate.astype(np.float64).sum(1)[:, None] * synth.bf16_bits_to_f32(x)
    assert P.rel_frob(P.out_as_f32(out, "bf16"), ref) <= 2e-2


def test_z0_and_k_equals_E():
    full_check(synth.Config("z0", T=100, d=128, I=64, N=7, Z=0, k=3, dtype="f32", seed=9),
               synth.host_inputs(synth.Config("z0", T=100, d=128, I=64, N=7, Z=0, k=3,
                                              dtype="f32", seed=9)))
    cfg = synth.Config("kE", T=50, d=64, I=32, N=5, Z=3, k=8, dtype="bf16", seed=10)
    _, cnt, _, _ = full_check(cfg, synth.host_inputs(cfg))
    assert (cnt == cfg.T).all()


@pytest.mark.parametrize("T", [700, 1700, 2600])
def test_single_hot_expert_spans_many_chunks(T):
    """Bias +10 on FFN expert 3: every token picks it, the rest of the slots
    route normally.  M_e = T rows in hot-expert chunks of 256 rows: 3, 7 or
    11 chunks (the last one 188, 164 or 40 rows, so up to three of its four
    64-token quarters are empty); above 8 chunks the tiles go in groups of 8
    chunks per row block."""
    cfg = synth.Config("hot", T=T, d=256, I=128, N=12, Z=4, k=3, dtype="bf16", seed=11)
    inp = synth.host_inputs(cfg)
    b = inp["bias"].copy()
    b[3] = 10.0
    _, cnt, idx, _ = full_check(cfg, inp, bias=b)
    assert cnt[3] == cfg.T and (idx[:, 0] == 3).all()


@pytest.mark.parametrize("dt,T", [("bf16", 2600), ("f32", 1700)])
def test_hot_experts_several_row_blocks_and_a_partial_chunk_group(dt, T):
    """Two FFN experts take every token (bias +10): 11 chunks each (bf16:
    hot-expert chunks of 256 rows, the last one 40; fp32: chunks of 160, the
    last one 100), i.e. one full group of 8 chunks per row block and a last,
    shorter group of 3; d = 640 and I = 384 give 3 gate/up row blocks of 128
    and 3 down row blocks of 256 (the last one half empty), so the grouped
    tile order runs over several row blocks."""
    cfg = synth.Config("hot2", T=T, d=640, I=384, N=6, Z=3, k=3, dtype=dt, seed=14)
    inp = synth.host_inputs(cfg)
    b = inp["bias"].copy()
    b[[1, 4]] = 10.0
    _, cnt, idx, _ = full_check(cfg, inp, bias=b)
    assert cnt[1] == cnt[4] == cfg.T


def test_hot_tiles_with_k_tails_and_partial_row_blocks():
    """bf16, every FFN expert above 160 rows (hot-expert tiles of 256 rows):
    d = 200 and I = 72 are not multiples of those tiles' 32-element K-step
    (the last step reads zeros past K), I is below one 128-row gate/up block
    and d below one 256-row down block (rows past them are clamped and
    their outputs dropped)."""
    cfg = synth.Config("hot_ktail", T=600, d=200, I=72, N=4, Z=2, k=3, dtype="bf16", seed=21)
    _, cnt, _, _ = full_check(cfg, synth.host_inputs(cfg), poison=True)
    assert (cnt[:cfg.N] > 160).sum() >= 2


def test_empty_and_single_token():
    cfg = synth.Config("one", T=1, d=64, I=16, N=4, Z=2, k=2, dtype="bf16", seed=12)
    full_check(cfg, synth.host_inputs(cfg))
    cfg0 = cfg.with_(T=0)
    dev = "cuda:0"
    x = torch.empty((0, cfg.d), dtype=torch.bfloat16, device=dev)
    w = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=dev)
    cnt = torch.full((cfg.E,), 7, dtype=torch.int32, device=dev)
    out, c, _, _ = moe.forward(x, w(cfg.E, cfg.d), torch.zeros(cfg.E, device=dev),
                               w(cfg.N, cfg.I, cfg.d), w(cfg.N, cfg.I, cfg.d),
                               w(cfg.N, cfg.d, cfg.I), cfg0.N, cfg0.Z, cfg0.k, counts=cnt)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.d) and (c.cpu() == 0).all()


def test_widths_not_multiples_of_8_timed_and_untimed_agree():
    """The zero-padded path under the stage timer (its copies run outside
    the timed stages): every stage recorded, outputs bit-identical to the
    untimed call."""
    cfg = ODD[0]
    inp = synth.host_inputs(cfg)
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)  # noqa: E731
    args = (t(inp["x"]), t(inp["W_router"]), torch.from_numpy(inp["bias"]).to(dev),
            t(inp["W_gate"]), t(inp["W_up"]), t(inp["W_down"]), cfg.N, cfg.Z, cfg.k)
    ref = moe.forward(*args)
    timer = moe.Timer(2)
    got = moe.forward(*args, timer=timer)
    n, ms = timer.read()
    timer.close()
    assert n == 1 and all(v > 0 for v in ms.values()), ms
    for u, v in zip(ref, got):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_stage_timer_records_every_stage():
    cfg = RAGGED[1]
    inp = synth.host_inputs(cfg)
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)
    timer = moe.Timer(4)
    for _ in range(3):
        moe.forward(t(inp["x"]), t(inp["W_router"]), torch.from_numpy(inp["bias"]).to(dev),
                    t(inp["W_gate"]), t(inp["W_up"]), t(inp["W_down"]), cfg.N, cfg.Z, cfg.k,
                    timer=timer)
    n, ms = timer.read()
    assert n == 3 and all(v >= 0 for v in ms.values()) and ms["gate_up"] > 0
    timer.close()
