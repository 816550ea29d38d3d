"""The seeded input generator, pinned to numpy's Philox, libm and torch's
bfloat16 cast.  CPU only."""
import ctypes
import math

import numpy as np
import pytest

import synth


def test_philox_matches_numpy():
    # numpy's Philox (4x64, 10 rounds) advances its counter before producing a
    # block, so its block for counter c is our block c+1.
    for n, k0, k1 in [(1, 0, 0), (2, 0, 3), (977, 12, 5), (2**40 + 3, 0, 4)]:
        bg = np.random.Philox(key=[k0, k1], counter=[n - 1, 0, 0, 0])
        assert (bg.random_raw(4) == synth.philox_block(n, k0, k1)).all()


def test_philox_known_answer():
    # Random123 known-answer vector for philox4x64-10, counter 0, key 0.
    assert [int(v) for v in synth.philox_block(0, 0, 0)] == [
        0x16554D9ECA36314C, 0xDB20FE9D672D0FDC, 0xD7E772CEE186176B, 0x7E68B68AEC7BA23B]


def test_transcendentals_match_libm():
    lib = synth._host_lib()
    for u in [2.0 ** -53, 1e-300, 1e-9, 0.1, 0.5, 0.70710678, 0.7071068, 0.999999, 1.0]:
        assert abs(lib.syn_ln_host(u) - math.log(u)) <= 4e-16 * max(1.0, abs(math.log(u)))
    for a in [0.0, 1e-20, 0.3, 2.0, 17.0, 73.5]:
        assert abs(lib.syn_sqrt_host(a) - math.sqrt(a)) <= 4e-16 * max(1.0, math.sqrt(a))
    s, c = ctypes.c_double(), ctypes.c_double()
    for v in np.linspace(0, 1, 4001)[:-1]:
        lib.syn_sincos_2pi_host(float(v), ctypes.byref(s), ctypes.byref(c))
        assert abs(s.value - math.sin(2 * math.pi * v)) < 2e-15
        assert abs(c.value - math.cos(2 * math.pi * v)) < 2e-15


def test_normal_moments():
    z = synth.host_normal((1 << 20,), 0, 0, 7, 1.0, "f32").astype(np.float64)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    # tail mass beyond 3 sigma against the normal law (0.27%)
    tail = (np.abs(z) > 3).mean()
    assert abs(tail - 0.0026998) < 5 * math.sqrt(0.0027 / n)


def test_slices_are_independent():
    full = synth.host_normal((40, 24), 0, 3, 4, 0.5, "bf16")
    part = synth.host_normal((7, 24), 11 * 24, 3, 4, 0.5, "bf16")
    assert (full[11:18] == part).all()
    odd = synth.host_normal((5,), 13, 3, 4, 0.5, "bf16")
    assert (full.reshape(-1)[13:18] == odd).all()
    u = synth.host_uniform(50, 0, 1, 2, -0.2, 0.2)
    assert (synth.host_uniform(9, 21, 1, 2, -0.2, 0.2) == u[21:30]).all()
    assert u.min() > -0.2 and u.max() <= np.float32(0.2)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    f32 = synth.host_normal((4096,), 0, 0, 9, 3.0, "f32")
    b16 = synth.host_normal((4096,), 0, 0, 9, 3.0, "bf16")
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (b16 == ref).all()
    assert (synth.f32_to_bf16_bits(f32) == ref).all()
    # ties to even on constructed halfway values
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (synth.f32_to_bf16_bits(vals) == ref).all()


def test_configs_follow_the_pages():
    import json, os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_model_config.json")))
    for name in ("prod", "decode", "skewed"):
        c = synth.CONFIGS[name]
        assert (c.d, c.I, c.N, c.Z, c.k) == (g["hidden_size"], g["ffn_expert_width"],
                                            g["ffn_experts_per_layer"], g["zero_experts_per_layer"],
                                            g["experts_per_token"])
