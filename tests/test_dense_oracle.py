"""Pin of the oracle's dense SwiGLU FFN (the dense block beside the MoE in
the shortcut-connected layer): against a float64 numpy re-derivation with
numpy's matmul (a library routine), and the closed form W3 = 0 => 0."""
import numpy as np

import oracle
import synth


def test_dense_ffn_matches_float64():
    cfg = synth.Config("dense", T=20, d=64, I=32, N=1, Z=1, k=1, dtype="bf16", seed=61)
    w = synth.host_dense(cfg, 96)
    out = oracle.dense_ffn(w["x_dense"], w["W1"], w["W3"], w["W2"], "bf16")
    f = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)  # noqa: E731
    x, w1, w3, w2 = f(w["x_dense"]), f(w["W1"]), f(w["W3"]), f(w["W2"])
    g = x @ w1.T
    ref = (g / (1.0 + np.exp(-g)) * (x @ w3.T)) @ w2.T
    err = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert err < 1e-5, err
    # swapping W1 and W3 changes the result (silu is applied to W1 x only)
    sw = oracle.dense_ffn(w["x_dense"], w["W3"], w["W1"], w["W2"], "bf16")
    assert np.linalg.norm(sw - ref) / np.linalg.norm(ref) > 1e-2
    zero = oracle.dense_ffn(w["x_dense"], w["W1"], np.zeros_like(w["W3"]), w["W2"], "bf16")
    assert not zero.any()
