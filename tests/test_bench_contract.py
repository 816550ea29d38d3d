"""bench.py's command-line contract that needs no GPU: a request for more
than one GPU is refused with a message (the path is single-GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps",
                        "1", "--warmup", "0"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_roofline_basis_follows_the_binding_bound():
    """The gate/up line is priced against MFMA where its FLOPs at the matrix
    peak outlast its bytes at the HBM peak (the small workload, whose four
    saturated experts carry thousands of tokens each) and against HBM at the
    production and decode shapes; the kernel label follows the dtype and the
    chunk height the library picks."""
    import numpy as np

    sys.path.insert(0, ROOT)
    import bench
    import synth

    def line(cfg, counts):
        alg = bench.algorithmic(cfg, counts)
        peak = bench.MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else bench.MFMA_F32_PEAK_TFLOPS
        return bench.dominant_roofline(cfg, alg["gate_up"], 1e-3, peak)

    # small: 4 experts with ~4094 tokens, 30 empty (the survey's simulation)
    c = np.zeros(synth.SMALL.E, np.int64)
    c[:4] = 4094
    c[4:34] = (synth.SMALL.T * synth.SMALL.k * 0.9 - 4 * 4094) // 30
    r = line(synth.SMALL, c)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and "gemm8w_kernel" in r["kernel"]
    prod = np.full(synth.PROD.E, 128, np.int64)
    r = line(synth.PROD, prod)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    r = line(synth.TINY, np.full(synth.TINY.E, 10, np.int64))
    assert "float" in r["kernel"] and "bf16" not in r["kernel"]
    assert "gemm_kernel<bf16,GATE_UP,1>" in line(synth.DECODE, np.full(synth.DECODE.E, 2))["kernel"]
