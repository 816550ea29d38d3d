"""Pins of the oracle's bias controller (the consumer of the forward's
per-expert counts).  The pages (LongCat-Flash summary, section 1 and section 2
"computation-budget control") call it a PID controller on an expert bias
that keeps the FFN / zero-expert selection ratio on target; the formula is
this project's reading (incremental PID on the per-token load error, see
oracle.c).  These tests tie it to hand-computed values and to its purpose:
driving the routing toward the target share."""
import numpy as np
import pytest

import oracle
import synth


def test_integral_step_by_hand():
    # e = (target - count) / T = (+0.5, -0.5, 0); bias += lr * e
    b, st = oracle.bias_update([10, 30, 20], [20, 20, 20], [0.0, 1.0, -1.0], T=20, lr=0.5)
    assert b.tolist() == [0.25, 0.75, -1.0] and st is None


def test_pid_terms_by_hand():
    """Three calls with errors 0.5, 0.25, -0.25 (dyadic, exact in fp32) and
    gains ki=1, kp=0.5, kd=0.25: steps 0.875, -0.0625, -0.5625."""
    st = np.zeros(2, np.float32)
    b = np.zeros(1, np.float32)
    steps = []
    for count in (2, 3, 5):  # T=4, target=4: e = (4 - count)/4
        nb, st = oracle.bias_update([count], [4.0], b, T=4, lr=1.0, ki=1.0, kp=0.5, kd=0.25,
                                    state=st)
        steps.append(float(nb[0] - b[0]))
        b = nb
    assert steps == [0.875, -0.0625, -0.5625]
    assert st.tolist() == [-0.25, 0.25]  # (e1, e2) after the third call
    assert b.tolist() == [0.25]


def test_no_history_means_pure_integral():
    """Without state the P and D terms vanish whatever their gains."""
    a, _ = oracle.bias_update([1, 7], [4, 4], [0, 0], T=8, lr=2.0, ki=1.0, kp=5.0, kd=3.0)
    c, _ = oracle.bias_update([1, 7], [4, 4], [0, 0], T=8, lr=2.0, ki=1.0)
    assert (a == c).all() and a.tolist() == [0.75, -0.75]


def test_on_target_leaves_bias_unchanged():
    rng = np.random.default_rng(0)
    E = 37
    cnt = rng.integers(0, 50, E).astype(np.int32)
    bias = rng.normal(size=E).astype(np.float32)
    st = np.zeros(2 * E, np.float32)
    b, st2 = oracle.bias_update(cnt, cnt.astype(np.float32), bias, T=100, lr=0.3, ki=1.0,
                                kp=0.7, kd=0.2, state=st)
    assert (b == bias).all() and (st2 == 0).all()


def test_sign_mode_moves_by_exactly_lr():
    b, _ = oracle.bias_update([0, 5, 9], [5, 5, 5], [0.5, 0.5, 0.5], T=10, lr=0.125, mode=1)
    assert b.tolist() == [0.625, 0.5, 0.375]


def test_closed_loop_drives_the_ffn_share_to_target():
    """Oracle routing + controller, repeated on one batch: the share of
    selections that go to FFN experts moves from its initial value to the
    target (here 0.75 of the k slots) and the FFN loads even out."""
    cfg = synth.Config("loop", T=512, d=64, I=16, N=8, Z=8, k=4, dtype="f32", seed=21,
                       bias_lo=0.0, bias_hi=0.0)
    x, wr = synth.host_x(cfg), synth.host_router(cfg)
    logits = oracle.router_logits(x, wr, "f32")
    E, T, k, N = cfg.E, cfg.T, cfg.k, cfg.N
    target = np.empty(E, np.float32)
    target[:N] = 0.75 * T * k / N
    target[N:] = 0.25 * T * k / cfg.Z
    bias = np.zeros(E, np.float32)
    st = np.zeros(2 * E, np.float32)

    def share(b):
        idx, _, _, _ = oracle.route_from_logits(logits, b, k)
        c = oracle.counts(idx, E)
        return c, c[:N].sum() / (T * k)

    c0, s0 = share(bias)
    lr = 0.02
    for it in range(200):
        c, _ = share(bias)
        bias, st = oracle.bias_update(c, target, bias, T=T, lr=lr * 0.99 ** it, ki=1.0, kp=0.5,
                                      state=st)
    c, s = share(bias)
    assert abs(s0 - 0.75) > 0.05, "the test needs a start away from the target"
    assert abs(s - 0.75) < 0.01
    ffn = c[:N] / (0.75 * T * k / N)
    assert ffn.min() > 0.8 and ffn.max() < 1.2
