"""moe_zc_forward_noalloc (the forward whose workspace is the library's
static per-GPU scratch array) against moe_zc_forward, through the C ABI.

Both run the same kernels, so the bar is bit-identity of every output
(out, counts, indices, gates), on calls in a row where the later ones are
smaller, so a stale remainder of an earlier call in the shared array would
show.  The decode shape (T = 128, d = 6144, I = 2048, 512 + 256 experts,
top-12) is the serving case this entry point is for."""
import ctypes

import numpy as np
import pytest

import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
moe = pytest.importorskip("zero_computation_expert_amd")
DEV = "cuda:0"


def _same(a, b):
    for u, v in zip(a, b):
        assert torch.equal(u, v) if u.dtype != torch.bfloat16 else \
            torch.equal(u.view(torch.int16), v.view(torch.int16))


def _pair(inp, N, Z, k, T):
    x = inp["x"][:T]
    args = (x, inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"], N, Z, k)
    nb = moe.workspace_bytes(T, x.shape[1], inp["W_gate"].shape[1], N, Z, k,
                             moe.BF16 if x.dtype == torch.bfloat16 else moe.F32)
    ws = torch.full((max(nb, 1),), 0xFF, dtype=torch.uint8, device=DEV)  # NaN bytes
    ref = moe.forward(*args, workspace=ws)
    got = moe.forward_noalloc(*args)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_equals_forward_on_calls_of_decreasing_size(dt):
    cfg = synth.Config("noalloc", T=600, d=512, I=384, N=24, Z=8, k=6, dtype=dt, seed=71,
                       bias_lo=-0.01, bias_hi=0.01)
    inp = synth.device_inputs(cfg, DEV)
    for T in (600, 97, 1):
        print(f"[noalloc] {dt} T={T}", flush=True)
        ref, got = _pair(inp, cfg.N, cfg.Z, cfg.k, T)
        _same(ref, got)
        assert int(got[1].sum()) == T * cfg.k


def test_noalloc_decode_shape_then_smaller():
    cfg = synth.DECODE
    inp = synth.device_inputs(cfg, DEV)
    for T in (cfg.T, 40):
        print(f"[noalloc] decode shape T={T}", flush=True)
        ref, got = _pair(inp, cfg.N, cfg.Z, cfg.k, T)
        _same(ref, got)
        assert np.isfinite(P.out_as_f32(P.to_np(got[0]), "bf16")).all()
    del inp
    torch.cuda.empty_cache()


def test_noalloc_widths_not_multiples_of_8():
    """The zero-padded path (copies with d and I rounded up to 8, in the
    shared array too), on two calls in a row, the second smaller."""
    cfg = synth.Config("noalloc_odd", T=200, d=100, I=36, N=6, Z=3, k=3, dtype="bf16", seed=72)
    h = synth.host_inputs(cfg)
    inp = {n: (torch.from_numpy(v).view(torch.bfloat16) if v.dtype == np.uint16
               else torch.from_numpy(v)).to(DEV) for n, v in h.items()}
    for T in (200, 31):
        print(f"[noalloc] d=100 I=36 T={T}", flush=True)
        ref, got = _pair(inp, cfg.N, cfg.Z, cfg.k, T)
        _same(ref, got)
        assert int(got[1].sum()) == T * cfg.k


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    big = moe.make_dims(8192, 6144, 2048, 512, 256, 12, moe.BF16)
    assert moe.lib().moe_zc_workspace_bytes(ctypes.byref(big)) > moe.SCRATCH_BYTES
    x = torch.empty(1, device=DEV)  # never reached: the size check comes first
    a = x.data_ptr()
    st = moe.lib().moe_zc_forward_noalloc(ctypes.byref(big), a, a, a, a, a, a, a, a, None, None,
                                          None)
    assert st == -6 and "scratch" in moe.status_string(st)
