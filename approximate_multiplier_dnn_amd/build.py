"""Build the HIP library (libapproxmul.so) in-tree for gfx950 with hipcc.

The library carries a stamp of the sources it was built from
(``approx_build_id()``: the first 16 hex digits of a SHA-256 over the files
of ``csrc/`` and the public header), so a stale binary can be told apart from
the sources beside it.
"""
import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libapproxmul.so")
CSRC = os.path.join(HERE, "csrc")
HEADER = os.path.join(ROOT, "include", "approx_mul.h")
SOURCES = [os.path.join(CSRC, f) for f in ("kernels.hip", "api.cpp", "lut_build.cpp")]

# Packed FP32 VALU instructions are disabled for every HIP translation unit.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def source_files():
    """Every file the library is built from, in a fixed order."""
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if not f.startswith("."))
    return files + [HEADER]


def source_hash():
    h = hashlib.sha256()
    for p in source_files():
        h.update(os.path.relpath(p, ROOT).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def build(extra=None, out=LIB):
    stamp = f'-DAPPROX_BUILD_ID="{source_hash()}"'
    cmd = ["/opt/rocm/bin/hipcc"] + HIPCC_FLAGS + [stamp] + (extra or []) + ["-o", out] + SOURCES
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build())
