"""Build the host (gcc) and device (hipcc, gfx950) generator libraries in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> None:
    host = os.path.join(HERE, "_synth_host.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared",
                    "-fPIC", "-o", host + ".tmp", os.path.join(CSRC, "synth_host.c")], check=True)
    os.replace(host + ".tmp", host)
    dev = os.path.join(HERE, "_synth_gpu.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-shared",
                        "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-o", dev + ".tmp", os.path.join(CSRC, "synth_gpu.hip")],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr)
    os.replace(dev + ".tmp", dev)


if __name__ == "__main__":
    build()
