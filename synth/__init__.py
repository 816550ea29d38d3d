"""Seeded synthetic inputs for the zero-computation-expert MoE forward.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds no step of the MoE method: it only draws the
activations ``x``, the router matrix ``W_router``, the expert matrices
``W_gate``/``W_up``/``W_down`` and the selection bias, from the counter-based
generator defined in ``synth/csrc/synth_rng.h`` (Philox4x64-10 + Box--Muller),
with a host build (``_synth_host.so``, gcc) and a device build
(``_synth_gpu.so``, hipcc) that give bit-identical values.

Workload shapes come from the LongCat-Flash model configuration (page
"LongCat-Flash" technical-report summary, section 2 "architecture", model
configuration paragraph: hidden size 6144, 512 FFN experts of width 2048, 256
zero-computation experts, 12 experts per token).  Values follow the stated
recipe: x ~ N(0, 1); every weight ~ N(0, 1/d_model); bias either uniform or a
fitted table (see ``tests/golden/fit_bias.py``, which computes those tables
with the oracle only).

Tensor ids (the Philox key's second word): x=0, W_router=1, bias=2,
W_gate=3, W_up=4, W_down=5.  Element ``flat`` of a tensor is its row-major
flat index, so any row range (one expert, a token slice) can be regenerated
on its own.
"""
from __future__ import annotations

import ctypes
import json
import math
import os
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_GOLDEN = os.path.join(os.path.dirname(_HERE), "tests", "golden")

TID_X, TID_WR, TID_BIAS, TID_WG, TID_WU, TID_WD = 0, 1, 2, 3, 4, 5
TID_DOUT = 6  # output gradient of the backward, N(0, 1) in the inputs' dtype
# the dense FFN block beside the MoE: its input x_dense ~ N(0, 1) and its
# SwiGLU matrices W1, W3 [I_dense, d], W2 [d, I_dense] ~ N(0, 1/d)
TID_XD, TID_D1, TID_D3, TID_D2 = 7, 8, 9, 10
DENSE_WIDTH = 12288  # the dense FFN path's intermediate width at the production shape


@dataclass(frozen=True)
class Config:
    """One workload: shapes, storage dtype and bias recipe.

    bias_kind: "uniform" (U(bias_lo, bias_hi) over all N+Z experts),
    "zero_offset" (0 for FFN experts, a fitted delta for zero experts, read
    from tests/golden/bias_prod.json), or "table" (a fitted per-expert
    vector read from tests/golden/<bias_file>).
    """

    name: str
    T: int
    d: int
    I: int
    N: int
    Z: int
    k: int
    dtype: str  # "f32" | "bf16"
    bias_kind: str = "uniform"
    bias_lo: float = -0.1
    bias_hi: float = 0.1
    bias_file: str = ""
    seed: int = 0

    @property
    def E(self) -> int:
        return self.N + self.Z

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


TINY = Config("tiny", T=64, d=128, I=64, N=8, Z=4, k=2, dtype="f32",
              bias_kind="uniform", bias_lo=-0.1, bias_hi=0.1)
SMALL = Config("small", T=4096, d=2048, I=1024, N=64, Z=32, k=6, dtype="bf16",
               bias_kind="uniform", bias_lo=-0.2, bias_hi=0.2)
PROD = Config("prod", T=8192, d=6144, I=2048, N=512, Z=256, k=12, dtype="bf16",
              bias_kind="zero_offset", bias_file="bias_prod.json")
DECODE = Config("decode", T=128, d=6144, I=2048, N=512, Z=256, k=12, dtype="bf16",
                bias_kind="zero_offset", bias_file="bias_prod.json")
SKEWED = Config("skewed", T=16384, d=6144, I=2048, N=512, Z=256, k=12, dtype="bf16",
                bias_kind="table", bias_file="bias_skewed.json")

CONFIGS = {c.name: c for c in (TINY, SMALL, PROD, DECODE, SKEWED)}


def sigma_weights(cfg: Config) -> float:
    return 1.0 / math.sqrt(float(cfg.d))


# --------------------------------------------------------------------------
# host build
# --------------------------------------------------------------------------
_host = None


def _host_lib():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "_synth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.syn_philox_block.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.POINTER(ctypes.c_uint64)]
        lib.syn_ln_host.restype = ctypes.c_double
        lib.syn_ln_host.argtypes = [ctypes.c_double]
        lib.syn_sqrt_host.restype = ctypes.c_double
        lib.syn_sqrt_host.argtypes = [ctypes.c_double]
        lib.syn_sincos_2pi_host.argtypes = [ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double)]
        lib.syn_normal_fill.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                        ctypes.c_double]
        lib.syn_uniform_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                         ctypes.c_double]
        lib.syn_bf16_from_f32.restype = ctypes.c_uint16
        lib.syn_bf16_from_f32.argtypes = [ctypes.c_float]
        _host = lib
    return _host


def philox_block(n: int, k0: int, k1: int) -> np.ndarray:
    out = (ctypes.c_uint64 * 4)()
    _host_lib().syn_philox_block(n, k0, k1, out)
    return np.array(list(out), dtype=np.uint64)


def host_normal(shape, first: int, seed: int, tid: int, sigma: float, dtype: str) -> np.ndarray:
    """Elements [first, first+prod(shape)) of normal tensor (seed, tid)."""
    count = int(np.prod(shape))
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        _host_lib().syn_normal_fill(out.ctypes.data, None, first, count, seed, tid, sigma)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        _host_lib().syn_normal_fill(None, out.ctypes.data, first, count, seed, tid, sigma)
    else:
        raise ValueError(dtype)
    return out


def host_uniform(count: int, first: int, seed: int, tid: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    _host_lib().syn_uniform_fill(out.ctypes.data, first, count, seed, tid, lo, hi)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ---- per-tensor host views of a workload ---------------------------------
def host_x(cfg: Config, t0: int = 0, nt: Optional[int] = None) -> np.ndarray:
    nt = cfg.T - t0 if nt is None else nt
    return host_normal((nt, cfg.d), t0 * cfg.d, cfg.seed, TID_X, 1.0, cfg.dtype)


def host_dout(cfg: Config, t0: int = 0, nt: Optional[int] = None) -> np.ndarray:
    """Output gradient rows [t0, t0+nt) for the backward (the inputs' dtype)."""
    nt = cfg.T - t0 if nt is None else nt
    return host_normal((nt, cfg.d), t0 * cfg.d, cfg.seed, TID_DOUT, 1.0, cfg.dtype)


def host_router(cfg: Config) -> np.ndarray:
    return host_normal((cfg.E, cfg.d), 0, cfg.seed, TID_WR, sigma_weights(cfg), cfg.dtype)


def host_expert(cfg: Config, which: str, e0: int, ne: int = 1) -> np.ndarray:
    """Experts [e0, e0+ne) of W_gate/W_up ([ne, I, d]) or W_down ([ne, d, I])."""
    per = cfg.I * cfg.d
    tid = {"gate": TID_WG, "up": TID_WU, "down": TID_WD}[which]
    shape = (ne, cfg.I, cfg.d) if which in ("gate", "up") else (ne, cfg.d, cfg.I)
    return host_normal(shape, e0 * per, cfg.seed, tid, sigma_weights(cfg), cfg.dtype)


def _golden(name: str) -> dict:
    path = os.path.join(_GOLDEN, name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} missing: run tests/golden/fit_bias.py (it uses the oracle)")
    with open(path) as f:
        return json.load(f)


def _hex_to_f32(h: str) -> np.float32:
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def host_bias(cfg: Config) -> np.ndarray:
    if cfg.bias_kind == "uniform":
        return host_uniform(cfg.E, 0, cfg.seed, TID_BIAS, cfg.bias_lo, cfg.bias_hi)
    if cfg.bias_kind == "zero_offset":
        g = _golden(cfg.bias_file)
        b = np.zeros(cfg.E, dtype=np.float32)
        b[cfg.N:] = _hex_to_f32(g["delta_f32_hex"])
        return b
    if cfg.bias_kind == "table":
        g = _golden(cfg.bias_file)
        b = np.array([_hex_to_f32(h) for h in g["bias_f32_hex"]], dtype=np.float32)
        if b.shape[0] != cfg.E:
            raise RuntimeError(f"bias table has {b.shape[0]} entries, expected {cfg.E}")
        return b
    raise ValueError(cfg.bias_kind)


def host_inputs(cfg: Config, experts: bool = True) -> dict:
    """All inputs on the host (x, W_router, bias and, if asked, all experts)."""
    out = {"x": host_x(cfg), "W_router": host_router(cfg), "bias": host_bias(cfg)}
    if experts:
        for w in ("gate", "up", "down"):
            out["W_" + w] = host_expert(cfg, w, 0, cfg.N) if cfg.N > 0 else None
    return out


# --------------------------------------------------------------------------
# device build (torch tensors are only storage here)
# --------------------------------------------------------------------------
_gpu = None


def _gpu_lib():
    global _gpu
    if _gpu is None:
        path = os.path.join(_HERE, "_synth_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.syn_normal_fill_device.restype = ctypes.c_int
        lib.syn_normal_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_double, ctypes.c_void_p]
        lib.syn_uniform_fill_device.restype = ctypes.c_int
        lib.syn_uniform_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                                ctypes.c_double, ctypes.c_void_p]
        _gpu = lib
    return _gpu


def device_normal(shape, first: int, seed: int, tid: int, sigma: float, dtype: str, device):
    import torch

    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = torch.empty(shape, dtype=tdt, device=device)
    n = out.numel()
    if n == 0:
        return out
    stream = torch.cuda.current_stream(device).cuda_stream
    if dtype == "f32":
        rc = _gpu_lib().syn_normal_fill_device(out.data_ptr(), None, first, n, seed, tid, sigma, stream)
    else:
        rc = _gpu_lib().syn_normal_fill_device(None, out.data_ptr(), first, n, seed, tid, sigma, stream)
    if rc != 0:
        raise RuntimeError(f"syn_normal_fill_device failed ({rc})")
    return out


def device_inputs(cfg: Config, device="cuda:0") -> dict:
    """All inputs generated directly in device memory (bit-identical to host_*)."""
    import torch

    sw = sigma_weights(cfg)
    out = {
        "x": device_normal((cfg.T, cfg.d), 0, cfg.seed, TID_X, 1.0, cfg.dtype, device),
        "W_router": device_normal((cfg.E, cfg.d), 0, cfg.seed, TID_WR, sw, cfg.dtype, device),
        "bias": torch.from_numpy(host_bias(cfg)).to(device),
    }
    for w, tid in (("gate", TID_WG), ("up", TID_WU), ("down", TID_WD)):
        shape = (cfg.N, cfg.I, cfg.d) if w != "down" else (cfg.N, cfg.d, cfg.I)
        out["W_" + w] = device_normal(shape, 0, cfg.seed, tid, sw, cfg.dtype, device)
    return out


def device_dout(cfg: Config, device="cuda:0"):
    """The output gradient of host_dout, generated in device memory."""
    return device_normal((cfg.T, cfg.d), 0, cfg.seed, TID_DOUT, 1.0, cfg.dtype, device)


def host_dense(cfg: Config, I_dense: int) -> dict:
    """x_dense [T, d] and the dense FFN matrices, in the inputs' dtype."""
    sw = sigma_weights(cfg)
    return {"x_dense": host_normal((cfg.T, cfg.d), 0, cfg.seed, TID_XD, 1.0, cfg.dtype),
            "W1": host_normal((I_dense, cfg.d), 0, cfg.seed, TID_D1, sw, cfg.dtype),
            "W3": host_normal((I_dense, cfg.d), 0, cfg.seed, TID_D3, sw, cfg.dtype),
            "W2": host_normal((cfg.d, I_dense), 0, cfg.seed, TID_D2, sw, cfg.dtype)}


def device_dense(cfg: Config, I_dense: int, device="cuda:0") -> dict:
    """The tensors of host_dense, generated in device memory."""
    sw = sigma_weights(cfg)
    return {"x_dense": device_normal((cfg.T, cfg.d), 0, cfg.seed, TID_XD, 1.0, cfg.dtype, device),
            "W1": device_normal((I_dense, cfg.d), 0, cfg.seed, TID_D1, sw, cfg.dtype, device),
            "W3": device_normal((I_dense, cfg.d), 0, cfg.seed, TID_D3, sw, cfg.dtype, device),
            "W2": device_normal((cfg.d, I_dense), 0, cfg.seed, TID_D2, sw, cfg.dtype, device)}
