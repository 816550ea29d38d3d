#!/usr/bin/env python3
"""Benchmark of the zero-computation-expert MoE forward on one MI355X.

One step = one moe_zc_forward call (router, top-k, dispatch, the two expert
GEMMs, combine) over one batch of synthetic tokens already resident in HBM.
Default workload: the production-shaped prefill layer (T=8192 tokens,
d=6144, 512 SwiGLU experts of width 2048, 256 zero experts, top-12, bf16).

Prints ONE JSON line with tokens/s, the per-stage times measured with HIP
events on the launch stream over the timed region, the roofline of the
dominant kernel and the CPU oracle's throughput on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 MI355X; % bf16 MFMA peak (prefill) / % HBM BW (decode)"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MFMA_F32_PEAK_TFLOPS = 157.3
MFMA_FP8_PEAK_TFLOPS = 5000.0  # dense fp8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prod", choices=["prod", "decode", "small", "skewed", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="oracle sample size (0: auto)")
    ap.add_argument("--fp8", action="store_true",
                    help="block-scaled FP8 experts (moe_zc_forward_fp8); a separate line, "
                         "not the bf16 headline")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_zc_backward (the block's backward with fp32 weight-gradient "
                         "accumulation); a separate line, not the forward headline")
    ap.add_argument("--scmoe", action="store_true",
                    help="time the shortcut-connected layer schedule: the MoE block and the "
                         "dense SwiGLU FFN (width 12288) serial, on two streams, and with the "
                         "MoE in two token chunks; a separate line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def algorithmic(cfg, counts, fp8=False):
    """Algorithmic FLOPs and HBM bytes of one step, and of each expert GEMM
    (fp8: expert weights and their activations one byte per element, plus
    one exponent byte per 128 x 128 weight block)."""
    import numpy as np

    s = 2 if cfg.dtype == "bf16" else 4
    ws = 1 if fp8 else s
    cnt = np.asarray(counts, dtype=np.int64)
    P = int(cnt[: cfg.N].sum())
    touched = int((cnt[: cfg.N] > 0).sum())
    T, d, I, E, k = cfg.T, cfg.d, cfg.I, cfg.E, cfg.k
    per_expert = d * I * ws + (d * I // (128 * 128) if fp8 else 0)
    step_bytes = (T * d * s * 2 + E * d * s + touched * 3 * per_expert + E * 8 + T * k * 8)
    step_flops = 6 * d * I * P + 2 * d * E * T
    gate_up = {"bytes": touched * 2 * per_expert + T * d * ws, "flops": 4 * d * I * P}
    down = {"bytes": touched * per_expert, "flops": 2 * d * I * P}
    # the other stages move each input and output once (fp32 logits, int32
    # indices, per-16-token-block histograms); their FLOPs are negligible
    nblk = (T + 15) // 16
    router = {"bytes": T * d * s + E * d * s + T * E * 4, "flops": 2 * d * E * T}
    topk = {"bytes": T * E * 4 + E * 4 + T * k * 8 + nblk * E * 4, "flops": 0}
    scan = {"bytes": 2 * nblk * E * 4 + E * 4 + (cfg.N + 1) * 8, "flops": 0}
    permute = {"bytes": T * k * 8 + nblk * cfg.N * 4 + P * 4, "flops": 0}
    if fp8:  # x quantized to E4M3 with one exponent per 128, and the exponents permuted
        permute["bytes"] += T * d * s + T * d + T * (d // 128) + P * (d // 128)
    combine = {"bytes": P * d * s + 2 * T * d * s + T * k * 8, "flops": 0}
    return {"P": P, "touched": touched, "step_bytes": step_bytes, "step_flops": step_flops,
            "gate_up": gate_up, "down": down, "router": router, "topk": topk, "scan": scan,
            "permute": permute, "combine": combine}


def gate_up_kernel_name(cfg, fp8=False):
    """The kernel the library launches for the gate/up stage of this
    workload: 160-token chunks (the 8-wave kernel) when experts average at
    least 96 rows, else 128 or 32 (the 4-wave kernel); fp32 always runs the
    4-wave kernel."""
    pmax = cfg.T * min(cfg.k, cfg.N)
    avg = pmax // cfg.N if cfg.N > 0 else 0
    nb = 5 if avg >= 96 else (4 if avg >= 24 else 1)
    if fp8:
        name = "gemm8f_w8_kernel<GATE_UP>" if nb == 5 else f"gemm8_kernel<GATE_UP,{nb}>"
        return name + " (FP8 gate/up GEMM + SwiGLU + [1,128] quantization of H)"
    if cfg.dtype == "bf16":
        name = "gemm8w_kernel<GATE_UP,5>" if nb == 5 else f"gemm_kernel<bf16,GATE_UP,{nb}>"
    else:
        name = f"gemm_kernel<float,GATE_UP,{nb}>"
    return name + " (gate/up GEMM + SwiGLU)"


def dominant_roofline(cfg, work, sec, peak_tf, fp8=False):
    """Roofline line of the gate/up GEMM, against the bound its algorithmic
    work binds on: MFMA when its FLOPs at the matrix peak take longer than
    its bytes at the HBM peak, else HBM."""
    t_mfma = work["flops"] / (peak_tf * 1e12)
    t_hbm = work["bytes"] / (HBM_PEAK_GBS * 1e9)
    base = {"kernel": gate_up_kernel_name(cfg, fp8), "algorithmic_bytes_per_launch": work["bytes"],
            "algorithmic_flops_per_launch": work["flops"], "avg_launch_ms": round(sec * 1e3, 4)}
    if t_mfma > t_hbm:
        tf = work["flops"] / sec / 1e12
        return {"bound": "mfma", "achieved": round(tf, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(tf / peak_tf, 4), **base}
    gbs = work["bytes"] / sec / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), **base}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


# HBM traffic of the dominant kernel, measured by rocprofv3 --pmc FETCH_SIZE
# and WRITE_SIZE in their own runs and kept in a committed summary together
# with the hash of the kernel source it was measured on; a summary taken on
# another version of the kernel is not reported.
KERNEL_SOURCES = {"gemm": ("gemm.hip", "gemm_common.h"),
                  "gemm8": ("gemm_fp8.hip", "gemm_common.h"),
                  "wgrad": ("gemm_bwd.hip", "gemm_common.h")}


def traffic_file(workload, kind):
    name = {"gemm": "gemm_gate_up", "gemm8": "gemm8_gate_up", "wgrad": "wgrad_gate_up"}[kind]
    return os.path.join(ROOT, "profiles", f"{name}_{workload}_hbm_traffic.txt")


def kernel_source_hash(kind="gemm"):
    """sha256 over the code of the kernel whose traffic is reported (gate/up
    GEMM: gemm.hip or gemm_fp8.hip; weight-gradient GEMM: gemm_bwd.hip; each
    with gemm_common.h), with comments and whitespace removed, so that only a
    change of code makes a measured traffic file stale."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        src = open(os.path.join(ROOT, "zero_computation_expert_amd", "csrc", f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)  # block comments
        src = re.sub(r"//[^\n]*", " ", src)  # line comments
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic(workload, kind="gemm"):
    path = traffic_file(workload, kind)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash(kind):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, dinp, ntok):
    """The oracle, as it is, on the first `ntok` tokens of the same workload."""
    import numpy as np

    import oracle
    import synth
    from tests import _parity as P

    t0 = time.time()
    x = synth.host_x(cfg, 0, ntok)
    wr = synth.host_router(cfg)
    bias = synth.host_bias(cfg)
    w = {n: P.to_np(dinp["W_" + n]) for n in ("gate", "up", "down")}  # generator's device copy
    prep = time.time() - t0
    t1 = time.time()
    oracle.forward(x, wr, bias, w["gate"], w["up"], w["down"], cfg.N, cfg.Z, cfg.k, cfg.dtype)
    dt = time.time() - t1
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens of the same workload (whole forward: "
                      f"router, top-k, experts, combine); {dt:.1f}s of oracle time on "
                      f"{threads} OpenMP threads of a {cpu_model()}, "
                      f"{prep:.1f}s input prep excluded"}


def calibrate_copy():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def backward_algorithmic(cfg, counts):
    """Algorithmic HBM bytes and FLOPs of the backward, per stage and per step:
    weights read once per touched expert, fp32 weight gradients read and
    written once, x / dout read, dx written (intermediates not counted)."""
    import numpy as np

    cnt = np.asarray(counts, dtype=np.int64)
    P = int(cnt[: cfg.N].sum())
    tch = int((cnt[: cfg.N] > 0).sum())
    T, d, I, E, k = cfg.T, cfg.d, cfg.I, cfg.E, cfg.k
    w2, g4 = d * I * 2, d * I * 4
    st = {
        "router": (T * d * 2 + E * d * 2, 2 * T * d * E),
        "recompute": (tch * 2 * w2 + T * d * 2, 4 * P * d * I),
        "dgrad_v": (tch * w2 + T * d * 2, 2 * P * d * I),
        "wgrad_down": (tch * 2 * g4, 2 * P * d * I),
        "wgrad_gate_up": (2 * tch * 2 * g4, 4 * P * d * I),
        "dgrad_x": (tch * 2 * w2, 4 * P * d * I),
        "dx": (E * d * 2 + 2 * T * d * 2, 2 * T * E * d),
        "wgrad_router": (2 * E * d * 4 + T * d * 2, 2 * T * E * d),
    }
    step_bytes = 3 * T * d * 2 + E * d * 2 + 3 * tch * w2 + 3 * tch * 2 * g4 + 2 * E * d * 4 + T * k * 8
    step_flops = 2 * 2 * T * d * E + (4 + 2 + 2 + 4 + 4) * P * d * I
    return {"P": P, "touched": tch, "stages": st, "step_bytes": step_bytes,
            "step_flops": step_flops}


def backward_cpu_baseline(cfg, inp, idx, gate, dout, ntok):
    """The oracle's per-token backward on the first ntok tokens (16 threads;
    the experts those tokens use are copied from the device generator's
    tensors, untimed).  It computes dx, the gate and router-logit gradients
    and the per-slot dg/du/h, but not the weight-gradient accumulation, so it
    overstates the oracle's rate for the whole backward."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth
    from tests import _parity as P

    t0 = time.time()
    x = P.to_np(inp["x"][:ntok])
    wr = P.to_np(inp["W_router"])
    idx_h, gate_h = idx[:ntok].cpu().numpy(), gate[:ntok].cpu().numpy()
    dout_h = synth.bf16_bits_to_f32(P.to_np(dout[:ntok]))
    used = sorted({int(e) for e in idx_h.ravel() if e < cfg.N})
    experts = {e: (P.to_np(inp["W_gate"][e]), P.to_np(inp["W_up"][e]), P.to_np(inp["W_down"][e]))
               for e in used}
    prep = time.time() - t0
    threads = min(16, ntok)

    def one(t):
        return oracle.token_backward(x[t], "bf16", wr, cfg.N, idx_h[t], gate_h[t], dout_h[t],
                                     {e: experts[e] for e in idx_h[t] if e < cfg.N})

    t1 = time.time()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(ntok)))
    sec = time.time() - t1
    return {"value": ntok / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {ntok} of {cfg.T} tokens, oracle per-token backward (dx, gate and "
                      f"router-logit gradients; weight-gradient accumulation not included, so "
                      f"this overstates the CPU rate); {sec:.1f}s on {threads} threads of a "
                      f"{cpu_model()}, {prep:.1f}s input copy excluded"}


def backward_bench(args, cfg, inp, dev):
    import torch

    import synth
    import zero_computation_expert_amd as moe

    if cfg.dtype != "bf16":
        print("the backward is bfloat16 only", file=sys.stderr)
        sys.exit(2)
    # routing from one untimed forward
    _, counts, idx, gate = moe.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"],
                                       inp["W_up"], inp["W_down"], cfg.N, cfg.Z, cfg.k)
    dout = synth.device_dout(cfg, dev)
    z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=dev)  # noqa: E731
    g = {"dW_router": z(cfg.E, cfg.d), "dW_gate": z(cfg.N, cfg.I, cfg.d),
         "dW_up": z(cfg.N, cfg.I, cfg.d), "dW_down": z(cfg.N, cfg.d, cfg.I)}
    nb = moe.backward_workspace_bytes(cfg.T, cfg.d, cfg.I, cfg.N, cfg.Z, cfg.k)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    dx = torch.empty_like(inp["x"])
    a = (inp["x"], inp["W_router"], inp["W_gate"], inp["W_up"], inp["W_down"], idx, gate, dout,
         cfg.N, cfg.Z)
    kw = dict(dx=dx, workspace=ws, **g)
    for _ in range(args.warmup):
        moe.backward(*a, **kw)
    torch.cuda.synchronize()
    timer = moe.Timer(max(1, args.steps), stages=moe.BWD_STAGES)
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        moe.backward(*a, **kw, timer=timer)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    ncalls, stage_ms = timer.read()
    timer.close()
    sa = {k: v / ncalls for k, v in stage_ms.items()}
    print(f"[bench] backward {args.steps} steps: {ms:.3f} ms/step; stages " +
          " ".join(f"{k}={v:.3f}" for k, v in sa.items()), file=sys.stderr, flush=True)
    alg = backward_algorithmic(cfg, counts.cpu().numpy())
    kernels = {}
    for name, (byt, fl) in alg["stages"].items():
        sec = sa[name] / 1e3
        kernels[name] = {"ms": round(sa[name], 4), "GB/s": round(byt / sec / 1e9, 1),
                         "TFLOP/s": round(fl / sec / 1e12, 1),
                         "hbm_frac": round(byt / sec / 1e9 / HBM_PEAK_GBS, 4),
                         "mfma_frac": round(fl / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # dominant kernel: the gate/up weight-gradient GEMM (two launches per
    # step, dW_gate then dW_up, equal bytes)
    per_launch = alg["stages"]["wgrad_gate_up"][0] // 2
    launch_ms = sa["wgrad_gate_up"] / 2
    gbs = per_launch / (launch_ms / 1e3) / 1e9
    step_s = ms / 1e3
    res = {
        "metric": "MoE-layer backward tokens/s at 1 MI355X (dx and fp32 weight gradients)",
        "value": round(cfg.T / step_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 operands, fp32 accumulation and fp32 weight gradients",
        "data": "synthetic (seeded Philox4x64 normals; random-init weights)",
        "config": {"workload": f"{cfg.name} backward: T={cfg.T} d={cfg.d} I={cfg.I} N={cfg.N} "
                               f"Z={cfg.Z} k={cfg.k} bf16",
                   "ffn_pairs": alg["P"], "touched_experts": alg["touched"]},
        "roofline": {"bound": "hbm", "kernel": "wgrad_kernel (dW_gate += dG^T X, dW_up += dU^T X; "
                     "fp32 read-modify-write of the gradient)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(cfg.name, "wgrad"),
                     "algorithmic_bytes_per_launch": per_launch,
                     "avg_launch_ms": round(launch_ms, 4)},
        "step_hbm_frac": round(alg["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(alg["step_flops"] / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "stages_ms": {k: round(v, 4) for k, v in sa.items()},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = backward_cpu_baseline(cfg, inp, idx, gate, dout,
                                                    args.cpu_tokens or 16)
    print(json.dumps(res), flush=True)


def scmoe_bench(args, cfg, inp, dev):
    import torch

    import synth
    import zero_computation_expert_amd as moe

    Id = synth.DENSE_WIDTH
    dn = synth.device_dense(cfg, Id, dev)
    s0 = torch.cuda.current_stream(dev)
    s1 = torch.cuda.Stream(device=dev)
    a1, b1 = moe.scmoe_workspace_bytes(cfg.T, cfg.d, cfg.I, cfg.N, cfg.Z, cfg.k, Id, 1)
    ws_moe = torch.empty(a1, dtype=torch.uint8, device=dev)
    ws_dense = torch.empty(b1, dtype=torch.uint8, device=dev)
    out_moe = torch.empty_like(inp["x"])
    out_dense = torch.empty_like(dn["x_dense"])
    counts = torch.empty((2, cfg.E), dtype=torch.int32, device=dev)

    def layer(nchunks, two):
        moe.scmoe_forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                          inp["W_down"], dn["x_dense"], dn["W1"], dn["W3"], dn["W2"], cfg.N,
                          cfg.Z, cfg.k, nchunks, s0, s1 if two else s0, out_moe=out_moe,
                          out_dense=out_dense, counts=counts[:nchunks], ws_moe=ws_moe,
                          ws_dense=ws_dense)

    def moe_only():
        moe.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                    inp["W_down"], cfg.N, cfg.Z, cfg.k, out=out_moe, counts=counts[0],
                    workspace=ws_moe, want_routing=False)

    def dense_only():
        moe.dense_ffn(dn["x_dense"], dn["W1"], dn["W3"], dn["W2"], out=out_dense,
                      workspace=ws_dense)

    def timed(fn):
        # each step starts both streams together and joins them at its end
        for _ in range(args.warmup):
            s1.wait_stream(s0)
            fn()
            s0.wait_stream(s1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s0)
        for _ in range(args.steps):
            s1.wait_stream(s0)
            fn()
            s0.wait_stream(s1)
        e1.record(s0)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms = {"moe_only": timed(moe_only), "dense_only": timed(dense_only),
          "serial": timed(lambda: layer(1, False)), "two_streams": timed(lambda: layer(1, True)),
          "two_chunks_serial": timed(lambda: layer(2, False)),
          "two_chunks_two_streams": timed(lambda: layer(2, True))}
    print("[bench] scmoe " + " ".join(f"{k}={v:.3f}" for k, v in ms.items()), file=sys.stderr,
          flush=True)
    # the headline is the fastest layer schedule; overlap_saving is what the
    # best overlapped schedule gains (negative: loses) against the serial one
    layers = ("serial", "two_streams", "two_chunks_serial", "two_chunks_two_streams")
    best = min(layers, key=lambda k: ms[k])
    best_overlap = min(("two_streams", "two_chunks_two_streams"), key=lambda k: ms[k])
    dense_flops = 6 * cfg.T * cfg.d * Id
    dense_tf = dense_flops / (ms["dense_only"] / 1e3) / 1e12
    res = {
        "metric": "shortcut-connected layer (MoE block + dense SwiGLU FFN) tokens/s at 1 MI355X",
        "value": round(cfg.T / (ms[best] / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms[best], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Philox4x64 normals; random-init weights)",
        "config": {"workload": f"{cfg.name} MoE (T={cfg.T} d={cfg.d} I={cfg.I} N={cfg.N} "
                               f"Z={cfg.Z} k={cfg.k}) + dense SwiGLU FFN width {Id}, bf16",
                   "schedule": best},
        "schedules_ms": {k: round(v, 4) for k, v in ms.items()},
        "overlap_schedule": best_overlap,
        "overlap_saving": round(1.0 - ms[best_overlap] / ms["serial"], 4),
        "roofline": {"bound": "mfma", "kernel": "dense FFN on gemm8w_kernel (gate/up + down)",
                     "achieved": round(dense_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dense_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_call": dense_flops,
                     "avg_call_ms": round(ms["dense_only"], 4)},
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    import numpy as np
    import torch

    import synth
    import zero_computation_expert_amd as moe

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    cfg = synth.CONFIGS[args.workload]
    dev = "cuda:0"
    t0 = time.time()
    inp = synth.device_inputs(cfg, dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs for {cfg.name} generated on device in {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)
    dt_code = moe.BF16 if cfg.dtype == "bf16" else moe.F32
    if args.backward:
        backward_bench(args, cfg, inp, dev)
        return
    if args.scmoe:
        scmoe_bench(args, cfg, inp, dev)
        return
    if args.fp8:
        # quantize the expert weights once, untimed ([128,128] blocks), and
        # drop the bf16 copies
        q = {}
        for w in ("W_gate", "W_up", "W_down"):
            q[w], q[w + "_exp"] = moe.quantize_fp8(inp[w], 128)
            inp[w] = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        nbytes = moe.workspace_bytes_fp8(cfg.T, cfg.d, cfg.I, cfg.N, cfg.Z, cfg.k)
        fwd = moe.forward_fp8
        args_fwd = (inp["x"], inp["W_router"], inp["bias"], q["W_gate"], q["W_gate_exp"],
                    q["W_up"], q["W_up_exp"], q["W_down"], q["W_down_exp"], cfg.N, cfg.Z, cfg.k)
    else:
        nbytes = moe.workspace_bytes(cfg.T, cfg.d, cfg.I, cfg.N, cfg.Z, cfg.k, dt_code)
        fwd = moe.forward
        args_fwd = (inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                    inp["W_down"], cfg.N, cfg.Z, cfg.k)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["x"])
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=dev)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=dev)
    kw = dict(out=out, counts=counts, topk_idx=idx, topk_gate=gate, workspace=ws)

    for _ in range(args.warmup):
        fwd(*args_fwd, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # headline: exactly `steps` calls back to back, each bracketed by HIP
    # events on the launch stream (no per-stage events inside); the median
    # call is the step time
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    ev0.record(stream)
    for a, b in evs:
        a.record(stream)
        fwd(*args_fwd, **kw)
        b.record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    calls_ms = [a.elapsed_time(b) for a, b in evs]
    ms = float(np.median(calls_ms))
    bracket_ms = ev0.elapsed_time(ev1) / args.steps
    # per-stage times: a second pass of `steps` calls through the library's
    # stage timer (HIP events after every kernel group, on the launch stream)
    timer = moe.Timer(max(1, args.steps))
    for _ in range(args.steps):
        fwd(*args_fwd, **kw, timer=timer)
    ncalls, stage_ms = timer.read()
    timer.close()
    stage_avg = {k: v / ncalls for k, v in stage_ms.items()}
    # cold: the same call after a 1 GiB write that evicts L2 and the MALL
    # (256 MB), the scrub outside the events
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold_ms = []
    for i in range(args.steps):
        scrub.fill_(i & 0xFF)
        a, b = evs[i]
        a.record(stream)
        fwd(*args_fwd, **kw)
        b.record(stream)
    torch.cuda.synchronize()
    cold_ms = [a.elapsed_time(b) for a, b in evs]
    del scrub
    print(f"[bench] {args.steps} steps: median {ms:.3f} ms/step (mean {bracket_ms:.3f}, "
          f"cold median {float(np.median(cold_ms)):.3f}); stages " +
          " ".join(f"{k}={v:.3f}" for k, v in stage_avg.items()), file=sys.stderr, flush=True)

    alg = algorithmic(cfg, counts.cpu().numpy(), fp8=args.fp8)
    gu_s = stage_avg["gate_up"] / 1e3
    peak_tf = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    expert_peak_tf = MFMA_FP8_PEAK_TFLOPS if args.fp8 else peak_tf
    roofline = dominant_roofline(cfg, alg["gate_up"], gu_s, expert_peak_tf, fp8=args.fp8)
    roofline["traffic"] = measured_traffic(cfg.name, "gemm8" if args.fp8 else "gemm")
    # every stage against the chip's peaks: HBM bytes for all, MFMA FLOPs for
    # the three contractions (top-k, the dispatch scans and permute, and
    # combine have no MFMA work)
    kernels = {}
    for name in ("router", "topk", "scan", "permute", "gate_up", "down", "combine"):
        sec = stage_avg[name] / 1e3
        a = alg[name]
        kernels[name] = {"ms": round(sec * 1e3, 4),
                         "GB/s": round(a["bytes"] / sec / 1e9, 1),
                         "hbm_frac": round(a["bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4)}
        if a["flops"]:
            pk = peak_tf if name == "router" else expert_peak_tf
            kernels[name]["TFLOP/s"] = round(a["flops"] / sec / 1e12, 1)
            kernels[name]["mfma_frac"] = round(a["flops"] / sec / 1e12 / pk, 4)
    step_s = ms / 1e3
    res = {
        "metric": METRIC,
        "value": round(cfg.T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "timing": {"ms_per_step": "median of the timed calls (HIP events around each call)",
                   "mean_ms": round(bracket_ms, 4), "min_ms": round(min(calls_ms), 4),
                   "max_ms": round(max(calls_ms), 4),
                   "cold_median_ms": round(float(np.median(cold_ms)), 4),
                   "cold_tokens_per_s": round(cfg.T / (float(np.median(cold_ms)) / 1e3), 1),
                   "cold": "each call after a 1 GiB scrub write (L2 and MALL evicted)"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8-e4m3 experts ([128,128] weight / [1,128] activation power-of-two "
                  "block scales), bf16 router and activations") if args.fp8 else cfg.dtype,
        "data": "synthetic (seeded Philox4x64 normals; random-init weights)",
        "config": {"workload": f"{cfg.name}: T={cfg.T} d={cfg.d} I={cfg.I} N={cfg.N} Z={cfg.Z} "
                               f"k={cfg.k} {cfg.dtype}" + (", FP8 experts" if args.fp8 else ""),
                   "T": cfg.T, "d": cfg.d, "I": cfg.I, "N": cfg.N, "Z": cfg.Z, "k": cfg.k,
                   "ffn_pairs": alg["P"], "touched_experts": alg["touched"]},
        "roofline": roofline,
        "step_hbm_frac": round(alg["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(alg["step_flops"] / step_s / 1e12 / expert_peak_tf, 4),
        # max(t_MFMA, t_HBM) / t: the fraction of the step's own roofline
        "step_roofline_frac": round(max(alg["step_bytes"] / 1e9 / HBM_PEAK_GBS,
                                        alg["step_flops"] / 1e12 / expert_peak_tf) / step_s, 4),
        "stages_ms": {k: round(v, 4) for k, v in stage_avg.items()},
        "kernels": kernels,
    }
    # bias controller (the step that consumes counts between forward calls),
    # timed on its own over 200 calls on the same stream
    target = torch.full((cfg.E,), float(cfg.T * cfg.k) / cfg.E, dtype=torch.float32, device=dev)
    bias_c = inp["bias"].clone()
    state = torch.zeros(2 * cfg.E, dtype=torch.float32, device=dev)
    moe.bias_update(counts, target, bias_c, cfg.T, 1e-3, 1.0, 0.5, 0.0, state, 0)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(200):
        moe.bias_update(counts, target, bias_c, cfg.T, 1e-3, 1.0, 0.5, 0.0, state, 0)
    ev1.record(stream)
    torch.cuda.synchronize()
    bu_us = ev0.elapsed_time(ev1) / 200 * 1e3
    res["bias_update"] = {"us_per_call": round(bu_us, 2), "experts": cfg.E,
                          "bytes_per_call": cfg.E * 32, "bound": "launch latency"}
    if not args.no_cpu_baseline and not args.fp8:  # the oracle baseline is the bf16 path's
        ntok = args.cpu_tokens or {"prod": 1536, "skewed": 1536, "decode": 128, "small": 4096,
                                   "tiny": 64}[cfg.name]
        res["cpu_baseline"] = cpu_baseline(cfg, inp, min(ntok, cfg.T))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
