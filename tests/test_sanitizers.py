"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds with the sanitizers on their host code, each exercised by the
existing CPU tests in a child process that preloads the matching runtime
(Python itself is not instrumented, so leak reports are off; any address or
undefined-behaviour report aborts the child):
  - the oracle (gcc -fsanitize=address,undefined), under the oracle pins;
  - the HIP library's host side (clang via hipcc, with -Xarch_host before
    each sanitizer flag so that no device code is instrumented), under the
    C-ABI tests: argument validation, workspace layout and error paths.
No GPU is touched: the ABI tests never pass validation.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(code, preload, timeout=900):
    env = dict(os.environ, LD_PRELOAD=preload, OMP_NUM_THREADS="4", **ENV)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "_oracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-shared", "-fPIC", "-o", so,
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    rt = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
import oracle
oracle._SO = {so!r}
oracle._lib = None
assert oracle._load()._name == {so!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                      "tests/test_oracle_pins.py", "tests/test_bias_controller.py",
                      "tests/test_dense_oracle.py", "tests/test_fullsize_helpers.py"]))
"""
    out = _child(code, rt)
    assert " passed" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    so = str(tmp_path / "_moe_zc_san.so")
    csrc = os.path.join(ROOT, "zero_computation_expert_amd", "csrc")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-shared-libsan", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", csrc,
           "-o", so] + sorted(glob.glob(os.path.join(csrc, "*.hip")))
    subprocess.run(cmd, check=True, capture_output=True)
    rts = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    assert rts, "clang's AddressSanitizer runtime not found"
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
import zero_computation_expert_amd as moe
moe.LIB_PATH = {so!r}
moe._lib = None
assert moe.lib()._name == {so!r}
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py"]))
"""
    out = _child(code, rts[-1])
    assert " passed" in out
