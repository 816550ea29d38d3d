"""Comparison rules between the HIP path and the CPU oracle (test helper).

Routing decisions are floating-point decisions of an integer result: both
sides take them in fp32, but they sum in different orders, so a token whose
k-th and (k+1)-th biased scores are closer than 1e-6 may legitimately pick a
different k-th expert.  Such tokens are excluded from the bit-exact index
and count checks; their outputs are compared against the oracle recomputed
with the GPU's own choice.  Indices are compared as sets (two experts inside
the top-k may be near-tied too); the order within a row is only checked to
be valid (non-increasing oracle score up to 1e-6).  In a near-tie row every
expert the GPU chose must score within 1e-6 of the oracle's k-th choice.

Tolerances: gates 1e-5 absolute; output relative Frobenius error 2e-2 for
bfloat16 and 1e-5 for fp32 over the compared tokens, and every single token
within 1.5x that bound (a localised error, such as a few wrong expert rows,
cannot hide in the aggregate).
"""
import numpy as np

import oracle
import synth

MARGIN = 1e-6
GATE_TOL = 1e-5
OUT_TOL = {"bf16": 2e-2, "f32": 1e-5}


def to_np(t):
    import torch

    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def out_as_f32(a, dt):
    return synth.bf16_bits_to_f32(a) if dt == "bf16" else np.asarray(a, np.float32)


def check_routing(cfg, bias, gpu_idx, gpu_gate, gpu_counts, ora_idx, ora_probs, ora_margin,
                  rows=None, scale=1.0):
    """rows: token indices the oracle arrays refer to (default: all); scale:
    the routed scale (gates are scale * p, an fp32 product, as in the
    oracle)."""
    T = gpu_idx.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    gi = gpu_idx[rows]
    gg = gpu_gate[rows]
    near = ora_margin < MARGIN
    ok = ~near
    # every GPU row: k distinct valid experts
    assert gi.min() >= 0 and gi.max() < cfg.E
    srt = np.sort(gi, axis=1)
    assert (np.diff(srt, axis=1) > 0).all(), "repeated expert in a row"
    # index sets bit-exact outside near-ties
    bad = np.nonzero((np.sort(ora_idx[ok], 1) != srt[ok]).any(1))[0]
    assert bad.size == 0, f"{bad.size} tokens route differently (first {rows[ok][bad[:5]]})"
    # order within a row: non-increasing oracle biased score
    s = ora_probs + bias[None, :]
    sc = np.take_along_axis(s, gi.astype(np.int64), 1)
    assert (np.diff(sc, axis=1) <= MARGIN).all(), "row not ordered by biased score"
    # near-tie rows: the GPU may swap experts only within the tie, so every
    # expert it chose scores at least the oracle's k-th score minus MARGIN
    if near.any():
        kth = np.take_along_axis(s[near], ora_idx[near][:, -1:].astype(np.int64), 1)
        assert (sc[near] >= kth - MARGIN).all(), "near-tie row picks an expert outside the tie"
    # gates: the oracle's probability of each GPU-chosen expert
    pg = np.float32(scale) * np.take_along_axis(ora_probs, gi.astype(np.int64), 1)
    gerr = float(np.abs(gg - pg).max()) if gg.size else 0.0
    assert gerr <= GATE_TOL, f"gate error {gerr}"
    # counts: bit-exact recount of the GPU's own indices
    assert (gpu_counts == np.bincount(gpu_idx.ravel(), minlength=cfg.E)).all()
    return {"near_ties": int(near.sum()), "gate_err": gerr}


def check_counts_against_oracle(cfg, gpu_idx, gpu_counts, ora_idx, ora_margin):
    """Full-T counts: equal to the oracle's once near-tie tokens are removed
    from both sides."""
    near = ora_margin < MARGIN
    g = gpu_counts.astype(np.int64) - np.bincount(gpu_idx[near].ravel(), minlength=cfg.E)
    o = np.bincount(ora_idx.ravel(), minlength=cfg.E) - np.bincount(ora_idx[near].ravel(),
                                                                     minlength=cfg.E)
    assert (g == o).all()
    if not near.any():
        assert (gpu_counts == np.bincount(ora_idx.ravel(), minlength=cfg.E)).all()


def rel_frob(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def worst_token_rel(got, ref):
    """Largest per-token relative error (rows of [T, d])."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return float((num / den).max()) if got.shape[0] else 0.0


def check_outputs(got, ref, dt):
    """Aggregate and per-token bounds; returns (aggregate, worst token)."""
    agg = rel_frob(got, ref)
    worst = worst_token_rel(got, ref)
    assert np.isfinite(got).all(), "non-finite output"
    assert agg <= OUT_TOL[dt], f"relative Frobenius error {agg}"
    assert worst <= 1.5 * OUT_TOL[dt], f"worst token relative error {worst}"
    return agg, worst


def reference_outputs(cfg, inp, gpu_idx, ora_probs, rows=None, scale=1.0):
    """Oracle outputs for `rows`, routed as the GPU routed them (identical to
    the oracle's own routing outside near-ties), gates = scale times the
    oracle probabilities (fp32)."""
    rows = np.arange(gpu_idx.shape[0]) if rows is None else np.asarray(rows)
    idx = gpu_idx[rows]
    gate = (np.float32(scale) *
            np.take_along_axis(ora_probs, idx.astype(np.int64), 1)).astype(np.float32)
    return oracle.combine_given_routing(inp["x"][rows], cfg.dtype, cfg.N, idx, gate,
                                        inp["W_gate"], inp["W_up"], inp["W_down"])
