"""Python binding of the MI355X zero-computation-expert MoE forward.

Argument marshalling only: every step of the forward runs in the HIP kernels
of ``_moe_zc.so`` behind the C ABI declared in ``include/moe_zc.h``.  Torch
tensors serve as device memory and torch's current stream as the HIP
stream.  There is no fallback: if the library is missing or no GPU is
visible, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_moe_zc.so")

F32, BF16 = 0, 1
STATUS = {0: "MOE_ZC_OK", -1: "MOE_ZC_EINVAL", -2: "MOE_ZC_EDTYPE", -3: "MOE_ZC_EALIGN",
          -4: "MOE_ZC_ENOSPC", -5: "MOE_ZC_EHIP", -6: "MOE_ZC_ESCRATCH"}
SCRATCH_BYTES = 64 << 20  # MOE_ZC_SCRATCH_BYTES: workspace limit of forward_noalloc
STAGES = ("router", "topk", "scan", "permute", "gate_up", "down", "combine")
BWD_STAGES = ("route", "router", "recompute", "dgrad_v", "router_bwd", "wgrad_down",
              "wgrad_gate_up", "dgrad_x", "dx", "wgrad_router")
MAX_STAGES = 10
EXPORTS = ("moe_zc_workspace_bytes", "moe_zc_forward", "moe_zc_status_string",
           "moe_zc_timer_create", "moe_zc_forward_timed", "moe_zc_timer_read",
           "moe_zc_timer_reset", "moe_zc_timer_destroy", "moe_zc_bias_update",
           "moe_zc_quantize_fp8", "moe_zc_workspace_bytes_fp8", "moe_zc_forward_fp8",
           "moe_zc_backward_workspace_bytes", "moe_zc_backward", "moe_zc_dense_workspace_bytes",
           "moe_zc_dense_ffn", "moe_zc_scmoe_workspace_bytes", "moe_zc_scmoe_forward",
           "moe_zc_forward_noalloc")


class MoeZcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("I", ctypes.c_int32),
                ("N", ctypes.c_int32), ("Z", ctypes.c_int32), ("k", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("routed_scale", ctypes.c_float)]


_lib = None


def lib():
    """Load ``_moe_zc.so`` (built by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        dims_p = ctypes.POINTER(Dims)
        L.moe_zc_workspace_bytes.restype = sz
        L.moe_zc_workspace_bytes.argtypes = [dims_p]
        fwd = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_zc_forward.restype = ctypes.c_int
        L.moe_zc_forward.argtypes = fwd
        L.moe_zc_forward_noalloc.restype = ctypes.c_int
        L.moe_zc_forward_noalloc.argtypes = fwd[:11] + [vp]
        L.moe_zc_forward_timed.restype = ctypes.c_int
        L.moe_zc_forward_timed.argtypes = fwd + [vp]
        L.moe_zc_status_string.restype = ctypes.c_char_p
        L.moe_zc_status_string.argtypes = [ctypes.c_int]
        L.moe_zc_timer_create.restype = ctypes.c_int
        L.moe_zc_timer_create.argtypes = [ctypes.c_int, ctypes.POINTER(vp)]
        L.moe_zc_timer_read.restype = ctypes.c_int
        L.moe_zc_timer_read.argtypes = [vp, ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_float)]
        L.moe_zc_timer_reset.restype = None
        L.moe_zc_timer_reset.argtypes = [vp]
        L.moe_zc_timer_destroy.restype = None
        L.moe_zc_timer_destroy.argtypes = [vp]
        L.moe_zc_quantize_fp8.restype = ctypes.c_int
        L.moe_zc_quantize_fp8.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
        L.moe_zc_workspace_bytes_fp8.restype = sz
        L.moe_zc_workspace_bytes_fp8.argtypes = [dims_p]
        L.moe_zc_forward_fp8.restype = ctypes.c_int
        L.moe_zc_forward_fp8.argtypes = [dims_p, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, sz, vp, vp]
        L.moe_zc_backward_workspace_bytes.restype = sz
        L.moe_zc_backward_workspace_bytes.argtypes = [dims_p]
        L.moe_zc_backward.restype = ctypes.c_int
        L.moe_zc_backward.argtypes = [dims_p] + [vp] * 14 + [sz, vp, vp]
        L.moe_zc_dense_workspace_bytes.restype = sz
        L.moe_zc_dense_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
        L.moe_zc_dense_ffn.restype = ctypes.c_int
        L.moe_zc_dense_ffn.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + [vp] * 6 \
            + [sz, vp]
        L.moe_zc_scmoe_workspace_bytes.restype = ctypes.c_int
        L.moe_zc_scmoe_workspace_bytes.argtypes = [dims_p, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.moe_zc_scmoe_forward.restype = ctypes.c_int
        L.moe_zc_scmoe_forward.argtypes = [dims_p, ctypes.c_int32, ctypes.c_int32] + [vp] * 15 \
            + [vp, sz, vp, sz, vp, vp]
        f32 = ctypes.c_float
        L.moe_zc_bias_update.restype = ctypes.c_int
        L.moe_zc_bias_update.argtypes = [ctypes.c_int32, ctypes.c_int64, vp, vp, vp, vp, f32, f32,
                                         f32, f32, ctypes.c_int32, vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_zc_status_string(status).decode()


def _check(status: int):
    if status != 0:
        raise MoeZcError(status, status_string(status))


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    return 99  # rejected by the library (MOE_ZC_EDTYPE)


def make_dims(T, d, I, N, Z, k, dtype: int, routed_scale: float = 1.0) -> Dims:
    return Dims(int(T), int(d), int(I), int(N), int(Z), int(k), int(dtype), float(routed_scale))


def workspace_bytes(T, d, I, N, Z, k, dtype: int) -> int:
    return int(lib().moe_zc_workspace_bytes(ctypes.byref(make_dims(T, d, I, N, Z, k, dtype))))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    p = t.data_ptr()
    return p if p != 0 else None


class Timer:
    """Per-stage HIP-event timer over up to ``max_calls`` forward (or, with
    ``stages=BWD_STAGES``, backward) calls."""

    def __init__(self, max_calls: int, stages=STAGES):
        h = ctypes.c_void_p()
        _check(lib().moe_zc_timer_create(int(max_calls), ctypes.byref(h)))
        self.handle = h
        self.stages = stages

    def read(self):
        """Synchronises on the events; returns (ncalls, {stage: total ms})."""
        n = ctypes.c_int()
        ms = (ctypes.c_float * MAX_STAGES)()
        _check(lib().moe_zc_timer_read(self.handle, ctypes.byref(n), ms))
        return n.value, dict(zip(self.stages, [float(v) for v in ms]))

    def reset(self):
        lib().moe_zc_timer_reset(self.handle)

    def close(self):
        if self.handle:
            lib().moe_zc_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def forward(x, W_router, bias, W_gate, W_up, W_down, N: int, Z: int, k: int, *,
            out=None, counts=None, topk_idx=None, topk_gate=None, workspace=None,
            stream=None, timer: Optional[Timer] = None, want_routing: bool = True,
            routed_scale: float = 1.0):
    """Runs moe_zc_forward on torch device tensors.

    x [T, d] and the weights share one dtype (float32 or bfloat16); W_gate and
    W_up are [N, I, d], W_down [N, d, I]; bias is float32 [N+Z].  Returns
    (out, counts, topk_idx, topk_gate); the last two are None unless
    ``want_routing``.  Output buffers and the workspace are allocated with
    torch when not given.
    """
    import torch

    T, d = x.shape
    I = W_gate.shape[1] if (W_gate is not None and N > 0) else 0
    dt = _dtype_code(x)
    dims = make_dims(T, d, I, N, Z, k, dt, routed_scale)
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    if counts is None:
        counts = torch.empty(N + Z, dtype=torch.int32, device=dev)
    if want_routing:
        if topk_idx is None:
            topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        if topk_gate is None:
            topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    if workspace is None:
        nbytes = int(lib().moe_zc_workspace_bytes(ctypes.byref(dims)))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    args = [ctypes.byref(dims), _ptr(x), _ptr(W_router), _ptr(bias), _ptr(W_gate), _ptr(W_up),
            _ptr(W_down), _ptr(out), _ptr(counts), _ptr(topk_idx), _ptr(topk_gate),
            _ptr(workspace), workspace.numel() * workspace.element_size(), stream]
    if timer is None:
        st = lib().moe_zc_forward(*args)
    else:
        st = lib().moe_zc_forward_timed(*args, timer.handle)
    _check(st)
    return out, counts, topk_idx, topk_gate


def forward_noalloc(x, W_router, bias, W_gate, W_up, W_down, N: int, Z: int, k: int, *,
                    out=None, counts=None, topk_idx=None, topk_gate=None, stream=None,
                    want_routing: bool = True, routed_scale: float = 1.0):
    """Runs moe_zc_forward_noalloc: as :func:`forward`, with the library's
    static per-GPU scratch array as the workspace (problems needing more than
    SCRATCH_BYTES of workspace raise MOE_ZC_ESCRATCH).  Output tensors not
    given are allocated here with torch; the library call itself allocates
    nothing."""
    import torch

    T, d = x.shape
    I = W_gate.shape[1] if (W_gate is not None and N > 0) else 0
    dims = make_dims(T, d, I, N, Z, k, _dtype_code(x), routed_scale)
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    if counts is None:
        counts = torch.empty(N + Z, dtype=torch.int32, device=dev)
    if want_routing:
        if topk_idx is None:
            topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        if topk_gate is None:
            topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _check(lib().moe_zc_forward_noalloc(ctypes.byref(dims), _ptr(x), _ptr(W_router), _ptr(bias),
                                        _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(out),
                                        _ptr(counts), _ptr(topk_idx), _ptr(topk_gate), stream))
    return out, counts, topk_idx, topk_gate


def bias_update(counts, target, bias, T: int, lr: float, ki: float = 1.0, kp: float = 0.0,
                kd: float = 0.0, state=None, mode: int = 0, stream=None):
    """Runs moe_zc_bias_update in place on torch device tensors: counts int32
    [E], target and bias float32 [E], state float32 [2E] or None."""
    import torch

    E = bias.numel()
    if stream is None:
        stream = torch.cuda.current_stream(bias.device).cuda_stream
    _check(lib().moe_zc_bias_update(int(E), int(T), _ptr(counts), _ptr(target), _ptr(bias),
                                    _ptr(state), float(lr), float(ki), float(kp), float(kd),
                                    int(mode), stream))
    return bias, state


# ---------------------------------------------------------------------------
# Block-scaled FP8 experts
# ---------------------------------------------------------------------------

def quantize_fp8(src, block_rows: int, q=None, scale_exp=None, stream=None):
    """moe_zc_quantize_fp8 on a torch device tensor [nmat, rows, K] or
    [rows, K] (float32 or bfloat16): returns (q uint8, same shape;
    scale_exp uint8 [nmat, rows/block_rows, K/128] or [rows/block_rows, K/128])."""
    import torch

    shape = tuple(src.shape)
    nmat, rows, K = (1,) + shape if len(shape) == 2 else shape
    if q is None:
        q = torch.empty(shape, dtype=torch.uint8, device=src.device)
    if scale_exp is None:
        sshape = (rows // block_rows, K // 128)
        scale_exp = torch.empty(sshape if len(shape) == 2 else (nmat,) + sshape,
                                dtype=torch.uint8, device=src.device)
    if stream is None:
        stream = torch.cuda.current_stream(src.device).cuda_stream
    _check(lib().moe_zc_quantize_fp8(_ptr(src), _dtype_code(src), int(nmat), int(rows), int(K),
                                     int(block_rows), _ptr(q), _ptr(scale_exp), stream))
    return q, scale_exp


def workspace_bytes_fp8(T, d, I, N, Z, k) -> int:
    return int(lib().moe_zc_workspace_bytes_fp8(ctypes.byref(make_dims(T, d, I, N, Z, k, BF16))))


def forward_fp8(x, W_router, bias, W_gate, W_gate_exp, W_up, W_up_exp, W_down, W_down_exp,
                N: int, Z: int, k: int, *, out=None, counts=None, topk_idx=None, topk_gate=None,
                workspace=None, stream=None, timer: Optional[Timer] = None,
                want_routing: bool = True, routed_scale: float = 1.0):
    """moe_zc_forward_fp8 on torch device tensors: x, W_router bfloat16; the
    expert matrices E4M3 bytes (uint8) with E8M0 exponents as returned by
    quantize_fp8(W, 128).  Returns (out, counts, topk_idx, topk_gate)."""
    import torch

    T, d = x.shape
    I = W_gate.shape[1] if (W_gate is not None and N > 0) else 0
    dims = make_dims(T, d, I, N, Z, k, _dtype_code(x), routed_scale)
    dev = x.device
    if out is None:
        out = torch.empty_like(x)
    if counts is None:
        counts = torch.empty(N + Z, dtype=torch.int32, device=dev)
    if want_routing:
        if topk_idx is None:
            topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        if topk_gate is None:
            topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    if workspace is None:
        nbytes = int(lib().moe_zc_workspace_bytes_fp8(ctypes.byref(dims)))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _check(lib().moe_zc_forward_fp8(
        ctypes.byref(dims), _ptr(x), _ptr(W_router), _ptr(bias), _ptr(W_gate), _ptr(W_gate_exp),
        _ptr(W_up), _ptr(W_up_exp), _ptr(W_down), _ptr(W_down_exp), _ptr(out), _ptr(counts),
        _ptr(topk_idx), _ptr(topk_gate), _ptr(workspace),
        workspace.numel() * workspace.element_size(), stream,
        timer.handle if timer is not None else None))
    return out, counts, topk_idx, topk_gate


# ---------------------------------------------------------------------------
# Backward of the block
# ---------------------------------------------------------------------------

def backward_workspace_bytes(T, d, I, N, Z, k) -> int:
    return int(lib().moe_zc_backward_workspace_bytes(
        ctypes.byref(make_dims(T, d, I, N, Z, k, BF16))))


def backward(x, W_router, W_gate, W_up, W_down, topk_idx, topk_gate, dout, N: int, Z: int, *,
             dx=None, dW_router=None, dW_gate=None, dW_up=None, dW_down=None, workspace=None,
             stream=None, timer: Optional[Timer] = None, routed_scale: float = 1.0):
    """moe_zc_backward on torch device tensors (bfloat16 x, weights and dout;
    the forward's topk_idx int32 / topk_gate float32).  Returns (dx, dW_router,
    dW_gate, dW_up, dW_down); the float32 weight gradients are accumulated
    into the given tensors, else into new zero tensors."""
    import torch

    T, d = x.shape
    k = topk_idx.shape[1]
    I = W_gate.shape[1] if (W_gate is not None and N > 0) else 0
    dims = make_dims(T, d, I, N, Z, k, _dtype_code(x), routed_scale)
    dev = x.device
    if dx is None:
        dx = torch.empty_like(x)
    z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=dev)  # noqa: E731
    if dW_router is None:
        dW_router = z(N + Z, d)
    if N > 0:
        if dW_gate is None:
            dW_gate = z(N, I, d)
        if dW_up is None:
            dW_up = z(N, I, d)
        if dW_down is None:
            dW_down = z(N, d, I)
    if workspace is None:
        nbytes = int(lib().moe_zc_backward_workspace_bytes(ctypes.byref(dims)))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _check(lib().moe_zc_backward(
        ctypes.byref(dims), _ptr(x), _ptr(W_router), _ptr(W_gate), _ptr(W_up), _ptr(W_down),
        _ptr(topk_idx), _ptr(topk_gate), _ptr(dout), _ptr(dx), _ptr(dW_router), _ptr(dW_gate),
        _ptr(dW_up), _ptr(dW_down), _ptr(workspace), workspace.numel() * workspace.element_size(),
        stream, timer.handle if timer is not None else None))
    return dx, dW_router, dW_gate, dW_up, dW_down


# ---------------------------------------------------------------------------
# Dense SwiGLU FFN and the two-stream ScMoE schedule
# ---------------------------------------------------------------------------

def dense_workspace_bytes(T, d, I_dense) -> int:
    return int(lib().moe_zc_dense_workspace_bytes(int(T), int(d), int(I_dense)))


def dense_ffn(x, W1, W3, W2, *, out=None, workspace=None, stream=None):
    """moe_zc_dense_ffn on bfloat16 device tensors: x [T, d], W1 / W3
    [I_dense, d], W2 [d, I_dense]; returns out [T, d]."""
    import torch

    T, d = x.shape
    Id = W1.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(dense_workspace_bytes(T, d, Id), 1), dtype=torch.uint8,
                                device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _check(lib().moe_zc_dense_ffn(int(T), int(d), int(Id), _ptr(x), _ptr(W1), _ptr(W3), _ptr(W2),
                                  _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), stream))
    return out


def scmoe_workspace_bytes(T, d, I, N, Z, k, I_dense, nchunks):
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().moe_zc_scmoe_workspace_bytes(ctypes.byref(make_dims(T, d, I, N, Z, k, BF16)),
                                              int(I_dense), int(nchunks), ctypes.byref(a),
                                              ctypes.byref(b)))
    return a.value, b.value


def scmoe_forward(x_moe, W_router, bias, W_gate, W_up, W_down, x_dense, W1, W3, W2, N: int,
                  Z: int, k: int, nchunks: int, stream_moe, stream_dense, *, out_moe=None,
                  out_dense=None, counts=None, topk_idx=None, topk_gate=None, ws_moe=None,
                  ws_dense=None, routed_scale: float = 1.0):
    """moe_zc_scmoe_forward: the MoE over x_moe (nchunks token chunks) on
    stream_moe and the dense FFN over x_dense on stream_dense (torch streams
    or raw handles).  Returns (out_moe, out_dense, counts [nchunks, N+Z],
    topk_idx, topk_gate)."""
    import torch

    T, d = x_moe.shape
    I = W_gate.shape[1] if (W_gate is not None and N > 0) else 0
    Id = W1.shape[0]
    dev = x_moe.device
    dims = make_dims(T, d, I, N, Z, k, _dtype_code(x_moe), routed_scale)
    if out_moe is None:
        out_moe = torch.empty_like(x_moe)
    if out_dense is None:
        out_dense = torch.empty_like(x_dense)
    if counts is None:
        counts = torch.empty((nchunks, N + Z), dtype=torch.int32, device=dev)
    if ws_moe is None or ws_dense is None:
        a, b = scmoe_workspace_bytes(T, d, I, N, Z, k, Id, nchunks)
        if ws_moe is None:
            ws_moe = torch.empty(max(a, 1), dtype=torch.uint8, device=dev)
        if ws_dense is None:
            ws_dense = torch.empty(max(b, 1), dtype=torch.uint8, device=dev)
    h = lambda s: s.cuda_stream if hasattr(s, "cuda_stream") else s  # noqa: E731
    _check(lib().moe_zc_scmoe_forward(
        ctypes.byref(dims), int(Id), int(nchunks), _ptr(x_moe), _ptr(W_router), _ptr(bias),
        _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(x_dense), _ptr(W1), _ptr(W3), _ptr(W2),
        _ptr(out_moe), _ptr(out_dense), _ptr(counts), _ptr(topk_idx), _ptr(topk_gate),
        _ptr(ws_moe), ws_moe.numel(), _ptr(ws_dense), ws_dense.numel(), h(stream_moe),
        h(stream_dense)))
    return out_moe, out_dense, counts, topk_idx, topk_gate
