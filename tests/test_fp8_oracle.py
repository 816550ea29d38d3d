"""Pins of the oracle's block-scaled FP8 expert path (test infrastructure).

The pages ask for DeepSeek-V3-style fine-grained quantization: activations
per [1,128] block, weights per [128,128] block (LongCat-Flash summary,
section 6, custom kernels).  The format (OCP E4M3), the rounding (nearest,
ties to even, saturating) and the scale rule (the smallest power of two >=
amax/448) are this project's readings; these tests tie the oracle to torch's float8_e4m3fn cast (a
library routine), to the format's arithmetic, to a float64 re-derivation of
the block-scaled forward and to the closed forms of the zero-expert paths."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def e4m3_values():
    """Every finite E4M3 magnitude (codes 0x00..0x7E)."""
    return np.array([oracle.e4m3_to_f32(q) for q in range(0x7F)], np.float32)


def test_decode_follows_the_format():
    v = e4m3_values()
    assert v[0] == 0 and v[1] == 2.0 ** -9 and v[8] == 2.0 ** -6 and v[0x38] == 1.0
    assert v[0x7E] == 448.0 and (np.diff(v) > 0).all()
    assert oracle.e4m3_to_f32(0x80 | 0x38) == -1.0


def test_encode_matches_torch_cast_and_rounds_ties_to_even():
    v = e4m3_values()
    mids = 0.5 * (v[1:] + v[:-1])
    cand = np.concatenate([v, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                           np.linspace(0, 463.9, 20001, dtype=np.float32)]).astype(np.float32)
    cand = np.concatenate([cand, -cand])
    ours = np.array([oracle.e4m3_from_f32(float(c)) for c in cand], np.uint8)
    ref = torch_e4m3(cand)
    zero = (ours & 0x7F) == 0  # +0 / -0 both acceptable for a zero result
    assert ((ours == ref) | (zero & ((ref & 0x7F) == 0))).all()
    # every code decodes and re-encodes to itself
    for q in range(0x7F):
        assert oracle.e4m3_from_f32(oracle.e4m3_to_f32(q)) == q


def test_saturates_at_448():
    for v in (448.0, 463.99, 464.0, 1e6):
        assert oracle.e4m3_from_f32(v) == 0x7E and oracle.e4m3_from_f32(-v) == 0xFE


@pytest.mark.parametrize("block_rows", [128, 1])
def test_block_quantization(block_rows):
    """Each block's scale is the smallest power of two >= amax/448, so its
    scaled largest magnitude lies in (224, 448]; every value is within half a step
    of the grid; the bytes equal torch's cast of v / scale; an all-zero
    block gets scale 1 and zeros."""
    rng = np.random.default_rng(block_rows)
    w = (rng.standard_normal((2, 256, 384)) * rng.choice([1e-3, 1.0, 30.0], (2, 256, 1)))
    w = w.astype(np.float32)
    w[1, :128, 128:256] = 0.0
    q, s = oracle.quantize_fp8(w, "f32", block_rows)
    assert q.shape == w.shape and s.shape == (2, 256 // block_rows, 3)
    deq = np.vectorize(oracle.e4m3_to_f32, otypes=[np.float32])(q & 0x7F)
    deq = np.where(q & 0x80, -deq, deq)
    for m in range(2):
        for rb in range(256 // block_rows):
            for kb in range(3):
                blk = (m, slice(rb * block_rows, (rb + 1) * block_rows), slice(kb * 128, kb * 128 + 128))
                v, sc = w[blk], s[m, rb, kb]
                amax = np.abs(v).max()
                if amax == 0:
                    assert sc == 1.0 and (q[blk] == 0).all()
                    continue
                r = np.float32(amax) / np.float32(448.0)
                mant, _ = np.frexp(sc)
                assert mant == 0.5 and sc >= r and sc / 2 < r  # power of two, smallest >= r
                assert 224.0 < amax / sc <= 448.0
                top = np.abs(deq[blk]).max()
                assert 224.0 <= top <= 448.0  # the scaled maximum may round down to 224
                ref = torch_e4m3(v / np.float32(sc))
                assert (q[blk] == ref).all()
                err = np.abs(deq[blk] * sc - v)
                assert (err <= np.maximum(np.abs(v) * 2.0 ** -4, sc * 2.0 ** -10) * 1.0001).all()


def _quant_rows_f64(v):
    """[1,128] quantization with torch's cast, returning dequantized float64."""
    v = np.asarray(v, np.float32)
    out = np.empty(v.shape, np.float64)
    for kb in range(v.shape[-1] // 128):
        blk = v[..., kb * 128:(kb + 1) * 128]
        amax = np.abs(blk).max(axis=-1, keepdims=True)
        r = (amax / np.float32(448.0)).astype(np.float32)
        sc = np.where(amax > 0, 2.0 ** np.ceil(np.log2(np.where(r > 0, r, 1.0).astype(np.float64))),
                      1.0).astype(np.float32)
        q = torch.from_numpy((blk / sc).astype(np.float32)).to(torch.float8_e4m3fn).float().numpy()
        out[..., kb * 128:(kb + 1) * 128] = q.astype(np.float64) * sc
    return out


def _dequant_w(q, s):
    vals = np.vectorize(oracle.e4m3_to_f32, otypes=[np.float64])(np.arange(256) & 0x7F)
    vals = np.where(np.arange(256) & 0x80, -vals, vals)
    deq = vals[q]
    return deq * np.repeat(np.repeat(s.astype(np.float64), 128, axis=1), 128, axis=2)


def _fp8_case(seed=31, T=24, d=256, I=256, N=4, Z=2, k=3):
    cfg = synth.Config("fp8", T=T, d=d, I=I, N=N, Z=Z, k=k, dtype="bf16", seed=seed)
    inp = synth.host_inputs(cfg)
    qg, sg = oracle.quantize_fp8(inp["W_gate"], "bf16", 128)
    qu, su = oracle.quantize_fp8(inp["W_up"], "bf16", 128)
    qd, sd = oracle.quantize_fp8(inp["W_down"], "bf16", 128)
    return cfg, inp, (qg, sg, qu, su, qd, sd)


def test_forward_fp8_matches_a_float64_rederivation():
    """Routing from the oracle, then experts recomputed in float64 with
    torch's FP8 cast for the activation quantization and numpy matmuls."""
    cfg, inp, w = _fp8_case()
    qg, sg, qu, su, qd, sd = w
    r = oracle.forward_fp8(inp["x"], inp["W_router"], inp["bias"], *w, cfg.N, cfg.Z, cfg.k, "bf16")
    x = synth.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    xh = _quant_rows_f64(x.astype(np.float32))
    Wg, Wu, Wd = _dequant_w(qg, sg), _dequant_w(qu, su), _dequant_w(qd, sd)
    ref = np.zeros_like(x)
    for t in range(cfg.T):
        for j in range(cfg.k):
            e, g = int(r["idx"][t, j]), float(r["gate"][t, j])
            if e >= cfg.N:
                ref[t] += g * x[t]
                continue
            gg, uu = Wg[e] @ xh[t], Wu[e] @ xh[t]
            h = gg / (1.0 + np.exp(-gg)) * uu
            hq = _quant_rows_f64(h.astype(np.float32)[None])[0]
            ref[t] += g * (Wd[e] @ hq)
    err = np.linalg.norm(r["out"] - ref) / np.linalg.norm(ref)
    assert err < 1e-4, err


def test_fp8_zero_expert_paths_are_exact():
    """W_up = 0: every FFN term vanishes, out = zsum * x (unquantized x)."""
    cfg, inp, w = _fp8_case(seed=32)
    qg, sg, qu, su, qd, sd = w
    qu0 = np.zeros_like(qu)
    r = oracle.forward_fp8(inp["x"], inp["W_router"], inp["bias"], qg, sg, qu0, su, qd, sd,
                           cfg.N, cfg.Z, cfg.k, "bf16")
    x = synth.bf16_bits_to_f32(inp["x"])
    zs = np.where(r["idx"] >= cfg.N, r["gate"], 0).sum(1, dtype=np.float32)
    assert np.array_equal(r["out"], (zs[:, None] * x).astype(np.float32))


def test_fp8_approximates_the_unquantized_forward():
    cfg, inp, w = _fp8_case(seed=33)
    r8 = oracle.forward_fp8(inp["x"], inp["W_router"], inp["bias"], *w, cfg.N, cfg.Z, cfg.k, "bf16")
    r16 = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                         inp["W_down"], cfg.N, cfg.Z, cfg.k, "bf16")
    assert (r8["idx"] == r16["idx"]).all()
    err = np.linalg.norm(r8["out"] - r16["out"]) / np.linalg.norm(r16["out"])
    assert 1e-3 < err < 0.1, err


def test_ffn_pairs_fp8_and_combine_slots_reproduce_the_fp8_forward():
    """The expert-major FP8 pieces used at full size give the FP8 forward's
    outputs bit for bit (same per-row activation quantization, same slot
    order)."""
    cfg, inp, w = _fp8_case(seed=34, T=19)
    qg, sg, qu, su, qd, sd = w
    r = oracle.forward_fp8(inp["x"], inp["W_router"], inp["bias"], *w, cfg.N, cfg.Z, cfg.k, "bf16")
    y = np.full((cfg.T, cfg.k, cfg.d), np.nan, np.float32)
    pairs = [(t, j) for t in range(cfg.T) for j in range(cfg.k) if r["idx"][t, j] < cfg.N]
    mats = [tuple(a[int(r["idx"][t, j])] for a in (qg, sg, qu, su, qd, sd)) for t, j in pairs]
    yy = oracle.ffn_pairs_fp8([inp["x"][t] for t, _ in pairs], "bf16", mats)
    for (t, j), row in zip(pairs, yy):
        y[t, j] = row
    out = oracle.combine_slots(inp["x"], "bf16", cfg.N, r["idx"], r["gate"], y)
    assert np.array_equal(out, r["out"])
