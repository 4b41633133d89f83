"""Build the HIP library (libapproxmul.so) in-tree for gfx950 with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libapproxmul.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "api.cpp", "lut_build.cpp")]
PROBE_SRC = os.path.join(HERE, "csrc", "lds_probe.hip")
PROBE = os.path.join(HERE, "lds_probe")

# Packed FP32 VALU instructions are disabled for every HIP translation unit.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(extra=None, out=LIB):
    cmd = ["/opt/rocm/bin/hipcc"] + HIPCC_FLAGS + (extra or []) + ["-o", out] + SOURCES
    subprocess.run(cmd, check=True)
    # the LDS lookup-rate probe behind the roofline numbers (bench.py --lds-probe)
    probe = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", PROBE, PROBE_SRC]
    subprocess.run(probe, check=True)
    return out


if __name__ == "__main__":
    print(build())
