"""CPU oracle for the zero-computation-expert MoE forward (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle.c`` (plain fp32 C,
built by :func:`build`) with numpy marshalling; it shares no code with the
HIP library and never calls it.

What it computes is documented, with the passages it follows, at the top of
``oracle.c``: router logits, softmax over all N+Z experts, bias added for
selection only, top-k with ties to the lower index, unbiased gates, SwiGLU
FFN experts, zero experts as identity, and the combine
``out = (sum of zero-slot gates) * x + sum_j gate_j * y_j``.

Pins (tests/test_oracle_pins.py) tie each function to something other than
itself: float64 library matmuls and softmax, brute-force top-k, the
closed forms of all-zero routing, Z = 0 (textbook top-k softmax MoE) and
identical experts, exact equivariance, and the model-size arithmetic printed
on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_oracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

F32, BF16 = 0, 1
_DT = {"f32": F32, "bf16": BF16}


def build() -> str:
    """Compile oracle.c into oracle/_oracle.so with gcc (always rebuilds)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
           "-o", _SO + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_router_logits.argtypes = [i64, i32, i32, vp, vp, i32, vp]
        lib.oracle_route_from_logits.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp,
                                                 ctypes.c_float]
        lib.oracle_counts.argtypes = [i64, i32, i32, vp, vp]
        lib.oracle_token_output.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp]
        lib.oracle_combine_given_routing.argtypes = [i64, i32, i32, i32, i32, vp, i32, vp, vp,
                                                     vp, vp, vp, vp]
        lib.oracle_ffn_pairs.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp]
        lib.oracle_combine_slots.argtypes = [i64, i32, i32, i32, vp, i32, vp, vp, vp, vp]
        lib.oracle_ffn_pairs_fp8.argtypes = [i64, i32, i32, i32] + [vp] * 8
        lib.oracle_forward.argtypes = [i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, vp, vp, ctypes.c_float]
        f32 = ctypes.c_float
        lib.oracle_bias_update.argtypes = [i32, i64, vp, vp, vp, vp, f32, f32, f32, f32, i32]
        lib.oracle_e4m3_from_f32.restype = ctypes.c_uint8
        lib.oracle_e4m3_from_f32.argtypes = [f32]
        lib.oracle_e4m3_to_f32.restype = f32
        lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        lib.oracle_quantize_fp8.argtypes = [vp, i32, i64, i32, i32, i32, vp, vp]
        lib.oracle_token_output_fp8.argtypes = [i32, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                                vp, vp, vp, vp]
        lib.oracle_combine_given_routing_fp8.argtypes = [i64, i32, i32, i32, i32, vp, i32, vp, vp,
                                                         vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_forward_fp8.argtypes = [i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                           vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float]
        lib.oracle_token_backward.argtypes = [i32, i32, i32, i32, i32, vp, i32] + [vp] * 13 + \
            [ctypes.c_float]
        lib.oracle_backward.argtypes = [i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                        vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float]
        lib.oracle_dense_ffn.argtypes = [i64, i32, i32, vp, i32, vp, vp, vp, vp]
        lib.oracle_expert_wgrad_row.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, i32,
                                                vp, vp, vp]
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _storage(a: np.ndarray, dt: str) -> np.ndarray:
    return _c(a, np.float32 if dt == "f32" else np.uint16)


def router_logits(x: np.ndarray, w_router: np.ndarray, dt: str) -> np.ndarray:
    x, w = _storage(x, dt), _storage(w_router, dt)
    T, d = x.shape
    E = w.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    _load().oracle_router_logits(T, d, E, _ptr(x), _ptr(w), _DT[dt], _ptr(out))
    return out


def route_from_logits(logits: np.ndarray, bias: np.ndarray, k: int, routed_scale: float = 1.0):
    """Returns idx [T,k] int32, gate [T,k] f32 (routed_scale * p of each
    selected expert), margin [T] f32, probs [T,E] f32 (unscaled)."""
    logits = _c(logits, np.float32)
    bias = _c(bias, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    margin = np.empty(T, dtype=np.float32)
    probs = np.empty((T, E), dtype=np.float32)
    _load().oracle_route_from_logits(T, E, k, _ptr(logits), _ptr(bias), _ptr(idx), _ptr(gate),
                                     _ptr(margin), _ptr(probs), float(routed_scale))
    return idx, gate, margin, probs


def counts(idx: np.ndarray, E: int) -> np.ndarray:
    idx = _c(idx, np.int32)
    T, k = idx.shape
    out = np.empty(E, dtype=np.int32)
    _load().oracle_counts(T, k, E, _ptr(idx), _ptr(out))
    return out


def token_output(x_row: np.ndarray, dt: str, N: int, idx_row, gate_row, experts: dict) -> np.ndarray:
    """Output of one token; ``experts[e] = (W_gate[e], W_up[e], W_down[e])`` for
    every FFN expert in ``idx_row`` (arrays in storage dtype)."""
    x_row = _storage(x_row, dt)
    d = x_row.shape[0]
    idx_row = _c(idx_row, np.int32)
    gate_row = _c(gate_row, np.float32)
    k = idx_row.shape[0]
    keep = []
    pg = (ctypes.c_void_p * k)()
    pu = (ctypes.c_void_p * k)()
    pd = (ctypes.c_void_p * k)()
    I = 1
    for j in range(k):
        e = int(idx_row[j])
        if e < N:
            g, u, dn = (_storage(a, dt) for a in experts[e])
            keep += [g, u, dn]
            I = g.shape[0]
            pg[j], pu[j], pd[j] = g.ctypes.data, u.ctypes.data, dn.ctypes.data
    out = np.empty(d, dtype=np.float32)
    _load().oracle_token_output(d, I, N, k, _ptr(x_row), _DT[dt], _ptr(idx_row), _ptr(gate_row),
                                pg, pu, pd, _ptr(out))
    return out


def combine_given_routing(x, dt, N, idx, gate, w_gate, w_up, w_down) -> np.ndarray:
    x = _storage(x, dt)
    T, d = x.shape
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    k = idx.shape[1]
    if N > 0:
        w_gate, w_up, w_down = (_storage(a, dt) for a in (w_gate, w_up, w_down))
        I = w_gate.shape[1]
    else:
        w_gate = w_up = w_down = None
        I = 1
    out = np.empty((T, d), dtype=np.float32)
    _load().oracle_combine_given_routing(T, d, I, N, k, _ptr(x), _DT[dt], _ptr(idx), _ptr(gate),
                                         _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out))
    return out


def _ptr_table(arrays):
    tab = (ctypes.c_void_p * max(1, len(arrays)))()
    for i, a in enumerate(arrays):
        tab[i] = a.ctypes.data
    return tab


def ffn_pairs(x_rows, dt: str, mats) -> np.ndarray:
    """Expert outputs of (token, FFN expert) pairs: ``x_rows[i]`` is pair i's
    token row (storage dtype, length d) and ``mats[i] = (W_gate[e], W_up[e],
    W_down[e])`` its expert's matrices.  Returns y [n, d] fp32, bit-identical
    to the per-slot expert output inside :func:`token_output`."""
    n = len(x_rows)
    rows = [_storage(r, dt) for r in x_rows]
    mm = [tuple(_storage(a, dt) for a in m) for m in mats]
    d = rows[0].shape[0] if n else 0
    I = mm[0][0].shape[0] if n else 1
    y = np.empty((n, d), dtype=np.float32)
    if n:
        _load().oracle_ffn_pairs(n, d, I, _DT[dt], _ptr_table(rows),
                                 _ptr_table([m[0] for m in mm]), _ptr_table([m[1] for m in mm]),
                                 _ptr_table([m[2] for m in mm]), _ptr(y))
    return y


def ffn_pairs_fp8(x_rows, dt: str, mats) -> np.ndarray:
    """As :func:`ffn_pairs` with FP8 experts: ``mats[i] = (qWg, sWg, qWu, sWu,
    qWd, sWd)`` (E4M3 bytes and fp32 block scales, as from
    :func:`quantize_fp8` with 128-row blocks); each token row is quantized per
    [1,128] first.  Bit-identical to one FFN slot of :func:`token_output_fp8`."""
    n = len(x_rows)
    rows = [_storage(r, dt) for r in x_rows]
    mm = [[_c(a, np.uint8 if i % 2 == 0 else np.float32) for i, a in enumerate(m)] for m in mats]
    d = rows[0].shape[0] if n else 0
    I = mm[0][0].shape[0] if n else 128
    y = np.empty((n, d), dtype=np.float32)
    if n:
        tabs = [_ptr_table([m[i] for m in mm]) for i in range(6)]
        _load().oracle_ffn_pairs_fp8(n, d, I, _DT[dt], _ptr_table(rows), *tabs, _ptr(y))
    return y


def combine_slots(x, dt: str, N: int, idx, gate, y_slots) -> np.ndarray:
    """Steps 4-5 given each FFN slot's expert output ``y_slots`` [T, k, d]
    (fp32; rows of zero slots are ignored): out = zsum * x + sum_j gate_j *
    y_j in ascending slot order, the combine of :func:`token_output`."""
    x = _storage(x, dt)
    T, d = x.shape
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    k = idx.shape[1]
    y_slots = _c(y_slots, np.float32)
    assert y_slots.shape == (T, k, d)
    out = np.empty((T, d), dtype=np.float32)
    _load().oracle_combine_slots(T, d, N, k, _ptr(x), _DT[dt], _ptr(idx), _ptr(gate),
                                 _ptr(y_slots), _ptr(out))
    return out


def forward(x, w_router, bias, w_gate, w_up, w_down, N: int, Z: int, k: int, dt: str,
            routed_scale: float = 1.0):
    """Whole forward. Returns dict(out, counts, idx, gate, margin)."""
    x = _storage(x, dt)
    w_router = _storage(w_router, dt)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E = N + Z
    if N > 0:
        w_gate, w_up, w_down = (_storage(a, dt) for a in (w_gate, w_up, w_down))
        I = w_gate.shape[1]
    else:
        w_gate = w_up = w_down = None
        I = 1
    out = np.empty((T, d), dtype=np.float32)
    cnt = np.empty(E, dtype=np.int32)
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    margin = np.empty(T, dtype=np.float32)
    _load().oracle_forward(T, d, I, N, Z, k, _DT[dt], _ptr(x), _ptr(w_router), _ptr(bias),
                           _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out), _ptr(cnt), _ptr(idx),
                           _ptr(gate), _ptr(margin), float(routed_scale))
    return {"out": out, "counts": cnt, "idx": idx, "gate": gate, "margin": margin}


def bias_update(counts, target, bias, T: int, lr: float, ki: float = 1.0, kp: float = 0.0,
                kd: float = 0.0, state=None, mode: int = 0):
    """Bias controller step (see oracle.c).  Returns (new bias, new state or
    None); the inputs are not modified."""
    counts = _c(counts, np.int32)
    target = _c(target, np.float32)
    b = np.array(bias, dtype=np.float32, copy=True)
    st = None if state is None else np.array(state, dtype=np.float32, copy=True)
    E = b.shape[0]
    assert counts.shape == (E,) and target.shape == (E,)
    assert st is None or st.shape == (2 * E,)
    _load().oracle_bias_update(E, T, _ptr(counts), _ptr(target), _ptr(b), _ptr(st),
                               float(lr), float(ki), float(kp), float(kd), int(mode))
    return b, st


# ---------------------------------------------------------------------------
# Block-scaled FP8 experts (see oracle.c for the readings)
# ---------------------------------------------------------------------------

def e4m3_from_f32(v: float) -> int:
    return int(_load().oracle_e4m3_from_f32(float(v)))


def e4m3_to_f32(q: int) -> float:
    return float(_load().oracle_e4m3_to_f32(int(q)))


def quantize_fp8(src, dt: str, block_rows: int):
    """src [nmat, rows, K] (or [rows, K]) in storage dtype -> (q uint8 same
    shape, scales float32 [nmat, rows/block_rows, K/128])."""
    a = _storage(src, dt)
    shape = a.shape
    if a.ndim == 2:
        a = a[None]
    nmat, rows, K = a.shape
    assert rows % block_rows == 0 and K % 128 == 0
    q = np.empty(a.shape, dtype=np.uint8)
    sc = np.empty((nmat, rows // block_rows, K // 128), dtype=np.float32)
    _load().oracle_quantize_fp8(_ptr(a), _DT[dt], nmat, rows, K, block_rows, _ptr(q), _ptr(sc))
    if len(shape) == 2:
        return q[0], sc[0]
    return q, sc


def token_output_fp8(x_row, dt: str, N: int, idx_row, gate_row, experts: dict) -> np.ndarray:
    """One token with FP8 experts; ``experts[e] = (qWg, sWg, qWu, sWu, qWd, sWd)``."""
    x_row = _storage(x_row, dt)
    d = x_row.shape[0]
    idx_row = _c(idx_row, np.int32)
    gate_row = _c(gate_row, np.float32)
    k = idx_row.shape[0]
    arrs = [(ctypes.c_void_p * k)() for _ in range(6)]
    keep = []
    I = 128
    for j in range(k):
        e = int(idx_row[j])
        if e < N:
            ex = [_c(a, np.uint8 if i % 2 == 0 else np.float32) for i, a in enumerate(experts[e])]
            keep += ex
            I = ex[0].shape[0]
            for i in range(6):
                arrs[i][j] = ex[i].ctypes.data
    out = np.empty(d, dtype=np.float32)
    _load().oracle_token_output_fp8(d, I, N, k, _ptr(x_row), _DT[dt], _ptr(idx_row),
                                    _ptr(gate_row), *arrs, _ptr(out))
    return out


def combine_given_routing_fp8(x, dt, N, idx, gate, qwg, swg, qwu, swu, qwd, swd) -> np.ndarray:
    x = _storage(x, dt)
    T, d = x.shape
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    k = idx.shape[1]
    qwg, qwu, qwd = (_c(a, np.uint8) for a in (qwg, qwu, qwd))
    swg, swu, swd = (_c(a, np.float32) for a in (swg, swu, swd))
    I = qwg.shape[1]
    out = np.empty((T, d), dtype=np.float32)
    _load().oracle_combine_given_routing_fp8(T, d, I, N, k, _ptr(x), _DT[dt], _ptr(idx),
                                             _ptr(gate), _ptr(qwg), _ptr(swg), _ptr(qwu),
                                             _ptr(swu), _ptr(qwd), _ptr(swd), _ptr(out))
    return out


def forward_fp8(x, w_router, bias, qwg, swg, qwu, swu, qwd, swd, N: int, Z: int, k: int, dt: str,
                routed_scale: float = 1.0):
    """Whole FP8-expert forward. Returns dict(out, counts, idx, gate, margin)."""
    x = _storage(x, dt)
    w_router = _storage(w_router, dt)
    bias = _c(bias, np.float32)
    T, d = x.shape
    E = N + Z
    qwg, qwu, qwd = (_c(a, np.uint8) for a in (qwg, qwu, qwd))
    swg, swu, swd = (_c(a, np.float32) for a in (swg, swu, swd))
    I = qwg.shape[1]
    out = np.empty((T, d), dtype=np.float32)
    cnt = np.empty(E, dtype=np.int32)
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float32)
    margin = np.empty(T, dtype=np.float32)
    _load().oracle_forward_fp8(T, d, I, N, Z, k, _DT[dt], _ptr(x), _ptr(w_router), _ptr(bias),
                               _ptr(qwg), _ptr(swg), _ptr(qwu), _ptr(swu), _ptr(qwd), _ptr(swd),
                               _ptr(out), _ptr(cnt), _ptr(idx), _ptr(gate), _ptr(margin),
                               float(routed_scale))
    return {"out": out, "counts": cnt, "idx": idx, "gate": gate, "margin": margin}


def token_backward(x_row, dt: str, w_router, N: int, idx_row, gate_row, dout_row,
                   experts: dict, routed_scale: float = 1.0) -> dict:
    """Backward of one token with given routing: dict(dx [d], dgate [k],
    dl [E] (router-logit gradient), h/dg/du [k, I] (rows of FFN slots)).
    ``experts[e] = (W_gate[e], W_up[e], W_down[e])`` for every FFN expert in
    ``idx_row``."""
    x_row = _storage(x_row, dt)
    w_router = _storage(w_router, dt)
    d = x_row.shape[0]
    E = w_router.shape[0]
    idx_row = _c(idx_row, np.int32)
    gate_row = _c(gate_row, np.float32)
    dout_row = _c(dout_row, np.float32)
    k = idx_row.shape[0]
    keep = []
    pg = (ctypes.c_void_p * k)()
    pu = (ctypes.c_void_p * k)()
    pd = (ctypes.c_void_p * k)()
    I = 1
    for j in range(k):
        e = int(idx_row[j])
        if e < N:
            g, u, dn = (_storage(a, dt) for a in experts[e])
            keep += [g, u, dn]
            I = g.shape[0]
            pg[j], pu[j], pd[j] = g.ctypes.data, u.ctypes.data, dn.ctypes.data
    dx = np.empty(d, dtype=np.float32)
    dgate = np.empty(k, dtype=np.float32)
    dl = np.empty(E, dtype=np.float32)
    h, dg, du = (np.zeros((k, I), dtype=np.float32) for _ in range(3))
    _load().oracle_token_backward(d, I, N, E, k, _ptr(x_row), _DT[dt], _ptr(w_router),
                                  _ptr(idx_row), _ptr(gate_row), _ptr(dout_row), pg, pu, pd,
                                  _ptr(dx), _ptr(dgate), _ptr(dl), _ptr(h), _ptr(dg), _ptr(du),
                                  float(routed_scale))
    return {"dx": dx, "dgate": dgate, "dl": dl, "h": h, "dg": dg, "du": du}


def backward(x, w_router, w_gate, w_up, w_down, idx, gate, dout, N: int, Z: int, dt: str,
             grads=None, routed_scale: float = 1.0) -> dict:
    """Whole backward with given routing (gate = routed_scale * p of each
    selected expert, as the forward gives it).  Returns dict(dx, dw_router,
    dw_gate, dw_up, dw_down); the weight gradients are accumulated into
    ``grads`` (a dict of fp32 arrays with those keys) when given, else into
    zeros."""
    x = _storage(x, dt)
    w_router = _storage(w_router, dt)
    T, d = x.shape
    E = N + Z
    idx = _c(idx, np.int32)
    gate = _c(gate, np.float32)
    dout = _c(dout, np.float32)
    k = idx.shape[1]
    if N > 0:
        w_gate, w_up, w_down = (_storage(a, dt) for a in (w_gate, w_up, w_down))
        I = w_gate.shape[1]
    else:
        w_gate = w_up = w_down = None
        I = 1
    if grads is None:
        grads = {"dw_router": np.zeros((E, d), np.float32),
                 "dw_gate": np.zeros((max(N, 0), I, d), np.float32),
                 "dw_up": np.zeros((max(N, 0), I, d), np.float32),
                 "dw_down": np.zeros((max(N, 0), d, I), np.float32)}
    g = {key: _c(grads[key], np.float32) for key in ("dw_router", "dw_gate", "dw_up", "dw_down")}
    dx = np.empty((T, d), dtype=np.float32)
    _load().oracle_backward(T, d, I, N, Z, k, _DT[dt], _ptr(x), _ptr(w_router), _ptr(w_gate),
                            _ptr(w_up), _ptr(w_down), _ptr(idx), _ptr(gate), _ptr(dout), _ptr(dx),
                            _ptr(g["dw_router"]), _ptr(g["dw_gate"]), _ptr(g["dw_up"]),
                            _ptr(g["dw_down"]), float(routed_scale))
    out = {"dx": dx}
    out.update(g)
    return out


def expert_wgrad_row(x_rows, dt: str, dout_rows, gates, wg, wu, wd, r: int) -> dict:
    """Row r of dW_gate[e] and dW_up[e] and column r of dW_down[e] from the n
    tokens routed to expert e (x_rows [n, d] in storage dtype, dout_rows
    [n, d] fp32, gates [n], tokens in ascending order)."""
    x_rows = _storage(x_rows, dt)
    n, d = x_rows.shape
    wg, wu, wd = (_storage(a, dt) for a in (wg, wu, wd))
    I = wg.shape[0]
    dout_rows = _c(dout_rows, np.float32)
    gates = _c(gates, np.float32)
    dwg, dwu, dwd = (np.empty(d, dtype=np.float32) for _ in range(3))
    _load().oracle_expert_wgrad_row(d, I, n, _ptr(x_rows), _DT[dt], _ptr(dout_rows), _ptr(gates),
                                    _ptr(wg), _ptr(wu), _ptr(wd), r, _ptr(dwg), _ptr(dwu),
                                    _ptr(dwd))
    return {"dw_gate_row": dwg, "dw_up_row": dwu, "dw_down_col": dwd}


def dense_ffn(x, w1, w3, w2, dt: str) -> np.ndarray:
    """The dense SwiGLU FFN: out [T, d] = W2 (silu(W1 x) * (W3 x)), fp32."""
    x = _storage(x, dt)
    T, d = x.shape
    w1, w3, w2 = (_storage(a, dt) for a in (w1, w3, w2))
    I = w1.shape[0]
    out = np.empty((T, d), dtype=np.float32)
    _load().oracle_dense_ffn(T, d, I, _ptr(x), _DT[dt], _ptr(w1), _ptr(w3), _ptr(w2), _ptr(out))
    return out
