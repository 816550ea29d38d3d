"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects every invalid argument before enqueueing work.

Every call here fails validation, so no kernel is ever launched (the fake
pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import zero_computation_expert_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_zc.h")

A = 1 << 20  # a 16- and 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_zc_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = moe.lib()
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = moe.status_string(code)
        assert s and s != "unknown status"
    assert moe.status_string(42) == "unknown status"


def call(dims, x=A, wr=2 * A, bias=3 * A, wg=4 * A, wu=5 * A, wd=6 * A, out=7 * A, counts=8 * A,
         idx=None, gate=None, ws=16 * A, ws_bytes=None):
    lib = moe.lib()
    if ws_bytes is None:
        ws_bytes = lib.moe_zc_workspace_bytes(ctypes.byref(dims)) if dims else 0
    dp = ctypes.byref(dims) if dims is not None else None
    st = lib.moe_zc_forward(dp, x, wr, bias, wg, wu, wd, out, counts, idx, gate, ws, ws_bytes, None)
    assert st != 0, "a test call passed validation: it would have launched work"
    return st


def D(T=64, d=128, I=64, N=8, Z=4, k=2, dtype=moe.BF16):
    return moe.make_dims(T, d, I, N, Z, k, dtype)


EINVAL, EDTYPE, EALIGN, ENOSPC = -1, -2, -3, -4


@pytest.mark.parametrize("dims,expect", [
    (D(dtype=7), EDTYPE),
    (D(T=-1), EINVAL),
    (D(k=0), EINVAL),
    (D(k=13), EINVAL),                       # k > N + Z
    (D(N=0, Z=0), EINVAL),                   # no experts
    (D(N=-1), EINVAL),
    (D(N=2000, Z=49, k=2), EINVAL),          # N + Z > 2048
    (D(N=100, Z=0, k=65), EINVAL),           # k > 64
    (D(d=0), EINVAL),
    (D(I=0), EINVAL),
    (D(T=1 << 28, k=8), EINVAL),             # T * k >= 2^31
    (D(T=1 << 20, d=1024, k=2), EINVAL),     # x is 2 GiB of bf16
    (D(I=1 << 17, d=8192), EINVAL),          # one expert matrix is 2 GiB
    (D(T=8, d=(1 << 22) + 8, I=8), EINVAL),  # d above 2^22
    (D(T=8, d=8, I=(1 << 22) + 8), EINVAL),  # I above 2^22
    (D(T=8, d=(1 << 22) + 1, I=8), EINVAL),  # d above 2^22, not a multiple of 8
])
def test_invalid_dims(dims, expect):
    assert moe.lib().moe_zc_workspace_bytes(ctypes.byref(dims)) == 0
    assert call(dims, ws_bytes=1 << 40) == expect


def test_widths_not_multiples_of_8_take_padded_workspace():
    # the forward runs such widths on zero-padded copies inside its workspace
    lib = moe.lib()
    ws = lambda dims: lib.moe_zc_workspace_bytes(ctypes.byref(dims))  # noqa: E731
    assert ws(D(d=100)) > ws(D(d=104)) > 0
    assert ws(D(I=60)) > ws(D(I=64)) > 0
    assert ws(D(d=1, I=1)) > 0 and ws(D(d=13, I=5, N=0, Z=4)) > 0
    # still validated before anything is enqueued
    assert call(D(d=100), ws_bytes=ws(D(d=104))) == ENOSPC
    assert call(D(d=100), x=A + 8) == EALIGN


def test_null_dims():
    assert moe.lib().moe_zc_workspace_bytes(None) == 0
    assert call(None, ws_bytes=1 << 40) == EINVAL


@pytest.mark.parametrize("kw,expect", [
    ({"counts": None}, EINVAL),
    ({"x": None}, EINVAL),
    ({"wr": None}, EINVAL),
    ({"bias": None}, EINVAL),
    ({"out": None}, EINVAL),
    ({"wg": None}, EINVAL),
    ({"wd": None}, EINVAL),
    ({"out": A + 64}, EINVAL),               # out overlaps x
    ({"x": A + 8}, EALIGN),
    ({"wu": 5 * A + 4}, EALIGN),
    ({"bias": 3 * A + 2}, EALIGN),
    ({"idx": 9 * A + 1}, EALIGN),
    ({"ws": None}, ENOSPC),
    ({"ws": 16 * A + 16}, EALIGN),           # workspace must be 256-byte aligned
])
def test_invalid_pointers(kw, expect):
    assert call(D(), **kw) == expect


def test_workspace_too_small():
    dims = D()
    need = moe.lib().moe_zc_workspace_bytes(ctypes.byref(dims))
    assert need > 0
    assert call(dims, ws_bytes=need - 1) == ENOSPC


def test_workspace_grows_with_tokens_and_covers_the_worst_case():
    lib = moe.lib()
    small = lib.moe_zc_workspace_bytes(ctypes.byref(D(T=64)))
    big = lib.moe_zc_workspace_bytes(ctypes.byref(D(T=4096)))
    assert big > small > 0
    # H and Y for every slot routed to an FFN expert, in bf16
    T, d, I, k = 4096, 128, 64, 2
    assert big >= T * k * (I + d) * 2


def test_weights_may_be_null_without_ffn_experts():
    # N = 0: null weights pass; the call still fails on the missing workspace
    assert call(D(N=0, Z=4, k=2), wg=None, wu=None, wd=None, ws=None, ws_bytes=0) == ENOSPC


def test_product_package_has_no_cpu_path():
    """The binding marshals arguments only: it imports neither the oracle nor
    numpy, and it has no compute of its own."""
    src = open(os.path.join(ROOT, "zero_computation_expert_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "import numpy" not in src
    for f in os.listdir(os.path.join(ROOT, "zero_computation_expert_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "zero_computation_expert_amd", "csrc", f)).read()


def bias_call(E=16, T=64, counts=A, target=2 * A, bias=3 * A, state=None, lr=0.1, ki=1.0,
              kp=0.0, kd=0.0, mode=0):
    st = moe.lib().moe_zc_bias_update(E, T, counts, target, bias, state, lr, ki, kp, kd, mode,
                                      None)
    assert st != 0, "a test call passed validation: it would have launched work"
    return st


@pytest.mark.parametrize("kw,expect", [
    (dict(E=0), EINVAL),
    (dict(E=-3), EINVAL),
    (dict(T=0), EINVAL),
    (dict(counts=None), EINVAL),
    (dict(target=None), EINVAL),
    (dict(bias=None), EINVAL),
    (dict(mode=2), EINVAL),
    (dict(lr=float("nan")), EINVAL),
    (dict(kp=float("inf")), EINVAL),
    (dict(bias=3 * A + 2), EALIGN),
    (dict(state=A + 1), EALIGN),
])
def test_bias_update_rejects(kw, expect):
    assert bias_call(**kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(dtype=5), EDTYPE),
    (dict(block_rows=64), EINVAL),
    (dict(rows=-1), EINVAL),
    (dict(K=200), EALIGN),
    (dict(rows=130), EALIGN),
    (dict(q=None), EINVAL),
    (dict(s=None), EINVAL),
    (dict(src=A + 8), EALIGN),
])
def test_quantize_fp8_rejects(kw, expect):
    a = dict(src=A, dtype=moe.BF16, nmat=2, rows=256, K=384, block_rows=128, q=2 * A, s=3 * A)
    a.update(kw)
    st = moe.lib().moe_zc_quantize_fp8(a["src"], a["dtype"], a["nmat"], a["rows"], a["K"],
                                       a["block_rows"], a["q"], a["s"], None)
    assert st == expect


def test_quantize_fp8_empty_is_ok():
    assert moe.lib().moe_zc_quantize_fp8(None, moe.BF16, 0, 128, 128, 128, None, None, None) == 0


def fp8_call(dims, exps=(9 * A, 10 * A, 11 * A), ws_bytes=None, **kw):
    lib = moe.lib()
    if ws_bytes is None:
        ws_bytes = lib.moe_zc_workspace_bytes_fp8(ctypes.byref(dims))
    st = lib.moe_zc_forward_fp8(ctypes.byref(dims), A, 2 * A, 3 * A, 4 * A, exps[0], 5 * A, exps[1],
                                6 * A, exps[2], 7 * A, 8 * A, None, None, 16 * A, ws_bytes, None,
                                None)
    assert st != 0, "a test call passed validation: it would have launched work"
    return st


def test_forward_fp8_rejects():
    assert fp8_call(D(T=64, d=256, I=128, dtype=moe.F32)) == EDTYPE
    assert fp8_call(D(T=64, d=200, I=128)) == EALIGN
    assert fp8_call(D(T=64, d=256, I=72)) == EALIGN
    assert fp8_call(D(T=64, d=256, I=128), exps=(9 * A, None, 11 * A)) == EINVAL
    assert fp8_call(D(T=64, d=256, I=128), ws_bytes=100) == ENOSPC
    assert moe.lib().moe_zc_workspace_bytes_fp8(ctypes.byref(D(T=64, d=200, I=128))) == 0
    assert (moe.lib().moe_zc_workspace_bytes_fp8(ctypes.byref(D(T=4096, d=256, I=128)))
            > moe.lib().moe_zc_workspace_bytes_fp8(ctypes.byref(D(T=64, d=256, I=128))))


def bwd_call(dims, ws_bytes=None, **kw):
    lib = moe.lib()
    if ws_bytes is None:
        ws_bytes = lib.moe_zc_backward_workspace_bytes(ctypes.byref(dims))
    p = {"x": A, "wr": 2 * A, "wg": 3 * A, "wu": 4 * A, "wd": 5 * A, "idx": 6 * A,
         "gate": 7 * A, "dout": 8 * A, "dx": 9 * A, "dwr": 10 * A, "dwg": 11 * A, "dwu": 12 * A,
         "dwd": 13 * A, "ws": 16 * A}
    p.update(kw)
    st = lib.moe_zc_backward(ctypes.byref(dims), p["x"], p["wr"], p["wg"], p["wu"], p["wd"],
                             p["idx"], p["gate"], p["dout"], p["dx"], p["dwr"], p["dwg"],
                             p["dwu"], p["dwd"], p["ws"], ws_bytes, None, None)
    assert st != 0, "a test call passed validation: it would have launched work"
    return st


@pytest.mark.parametrize("kw,expect", [
    ({"x": None}, EINVAL),
    ({"idx": None}, EINVAL),
    ({"gate": None}, EINVAL),
    ({"dout": None}, EINVAL),
    ({"dx": None}, EINVAL),
    ({"dwr": None}, EINVAL),
    ({"dwd": None}, EINVAL),
    ({"dx": A + 64}, EINVAL),                # dx overlaps x
    ({"dx": 8 * A + 32}, EINVAL),            # dx overlaps dout
    ({"dout": 8 * A + 8}, EALIGN),
    ({"dwg": 11 * A + 2}, EALIGN),
    ({"ws": None}, ENOSPC),
    ({"ws": 16 * A + 16}, EALIGN),
])
def test_backward_rejects(kw, expect):
    assert bwd_call(D(), **kw) == expect


def test_backward_rejects_dims():
    assert bwd_call(D(dtype=moe.F32)) == EDTYPE
    assert bwd_call(D(d=100)) == EALIGN
    assert bwd_call(D(), ws_bytes=100) == ENOSPC
    assert moe.lib().moe_zc_backward_workspace_bytes(ctypes.byref(D(dtype=moe.F32))) == 0
    big = moe.lib().moe_zc_backward_workspace_bytes(ctypes.byref(D(T=4096)))
    assert big > moe.lib().moe_zc_backward_workspace_bytes(ctypes.byref(D(T=64))) > 0


def test_dense_ffn_rejects():
    lib = moe.lib()
    need = lib.moe_zc_dense_workspace_bytes(64, 128, 256)
    assert need > 0 and lib.moe_zc_dense_workspace_bytes(64, 100, 256) == 0

    def dense(T=64, d=128, Id=256, x=A, w1=2 * A, w3=3 * A, w2=4 * A, out=5 * A, ws=16 * A,
              nb=None):
        st = lib.moe_zc_dense_ffn(T, d, Id, x, w1, w3, w2, out, ws, need if nb is None else nb,
                                  None)
        assert st != 0, "a test call passed validation: it would have launched work"
        return st

    assert dense(d=100) == EALIGN
    assert dense(Id=60) == EALIGN
    assert dense(T=8, d=8, Id=(1 << 22) + 8) == EINVAL   # width above 2^22
    assert dense(x=None) == EINVAL
    assert dense(out=A + 32) == EINVAL   # out overlaps x
    assert dense(w2=4 * A + 4) == EALIGN
    assert dense(nb=need - 1) == ENOSPC
    assert dense(ws=16 * A + 16) == EALIGN


def test_scmoe_rejects():
    lib = moe.lib()
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.moe_zc_scmoe_workspace_bytes(ctypes.byref(D()), 256, 3, ctypes.byref(a),
                                            ctypes.byref(b)) == EINVAL
    assert lib.moe_zc_scmoe_workspace_bytes(ctypes.byref(D(dtype=moe.F32)), 256, 2,
                                            ctypes.byref(a), ctypes.byref(b)) == EDTYPE
    assert lib.moe_zc_scmoe_workspace_bytes(ctypes.byref(D()), 256, 2, ctypes.byref(a),
                                            ctypes.byref(b)) == 0
    one, two = a.value, ctypes.c_size_t()
    assert lib.moe_zc_scmoe_workspace_bytes(ctypes.byref(D()), 256, 1, ctypes.byref(two),
                                            ctypes.byref(b)) == 0
    assert two.value > one  # two chunks need a workspace of half the tokens

    def sc(nchunks=2, counts=8 * A, ws_moe_bytes=None, x_dense=20 * A, out_dense=21 * A):
        st = lib.moe_zc_scmoe_forward(ctypes.byref(D()), 256, nchunks, A, 2 * A, 3 * A, 4 * A,
                                      5 * A, 6 * A, x_dense, 22 * A, 23 * A, 24 * A, 7 * A,
                                      out_dense, counts, None, None, 16 * A,
                                      one if ws_moe_bytes is None else ws_moe_bytes, 32 * A,
                                      b.value, None, None)
        assert st != 0, "a test call passed validation: it would have launched work"
        return st

    assert sc(nchunks=0) == EINVAL
    assert sc(counts=None) == EINVAL
    assert sc(ws_moe_bytes=one - 1) == ENOSPC
    assert sc(out_dense=7 * A + 64) == EINVAL    # overlaps out_moe
    assert sc(x_dense=None) == EINVAL


@pytest.mark.parametrize("dims,expect", [
    (D(dtype=7), EDTYPE),
    (D(k=0), EINVAL),
    (D(d=0), EINVAL),
    (D(T=8192, d=6144, I=2048, N=512, Z=256, k=12), -6),  # needs ~1.5 GB > the static scratch
    (D(T=4096, d=1000, I=1000, N=64, Z=32, k=6), -6),     # padded copies of every expert
])
def test_noalloc_rejects_before_touching_the_device(dims, expect):
    """moe_zc_forward_noalloc validates like moe_zc_forward and rejects a
    problem whose workspace exceeds MOE_ZC_SCRATCH_BYTES with its own code,
    before any HIP call (none can succeed here: there is no GPU)."""
    st = moe.lib().moe_zc_forward_noalloc(ctypes.byref(dims), A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A,
                                          7 * A, 8 * A, None, None, None)
    assert st == expect


def test_noalloc_validates_pointers_first():
    lib = moe.lib()
    dims = D()
    assert lib.moe_zc_workspace_bytes(ctypes.byref(dims)) <= moe.SCRATCH_BYTES
    assert lib.moe_zc_forward_noalloc(ctypes.byref(dims), None, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A,
                                      7 * A, 8 * A, None, None, None) == EINVAL
    assert lib.moe_zc_forward_noalloc(ctypes.byref(dims), A + 2, 2 * A, 3 * A, 4 * A, 5 * A,
                                      6 * A, 7 * A, 8 * A, None, None, None) == EALIGN


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan"), float("inf")])
def test_routed_scale_must_be_finite_and_positive(scale):
    dims = moe.make_dims(64, 128, 64, 8, 4, 2, moe.BF16, scale)
    assert moe.lib().moe_zc_workspace_bytes(ctypes.byref(dims)) == 0
    assert call(dims, ws_bytes=1 << 40) == EINVAL
