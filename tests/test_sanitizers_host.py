"""The host code built with AddressSanitizer and UndefinedBehaviorSanitizer
(host compilers only, no GPU): the oracle (oracle/oracle.c), the library's
table builder (csrc/lut_build.cpp) and the M = 8 copy choice (csrc/replica.h)
run under tests/sanitizer_driver.cpp, which drives them over every table
width, odd and padded shapes, transposes, Conv2D geometries with strides and
paddings, sampled outputs and chunked FP32 sums. Any sanitizer report ends
the run with a non-zero status; the driver also checks that the two table
builders agree."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("host compilers not available")
    d = tmp_path_factory.mktemp("san")
    obj = str(d / "oracle.o")
    exe = str(d / "sanitizer_driver")
    subprocess.run(["gcc", "-std=c99", "-ffp-contract=off", "-fno-fast-math", *SAN, "-c",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", obj], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wno-unknown-pragmas", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    *SAN, os.path.join(ROOT, "tests", "sanitizer_driver.cpp"),
                    os.path.join(ROOT, "approximate_multiplier_dnn_amd", "csrc", "lut_build.cpp"), obj,
                    "-o", exe, "-lm"], check=True)
    return exe


def test_host_code_under_address_and_undefined_behaviour_sanitizers(driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "0 failures" in r.stdout
