"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every function of include/approx_mul.h, its table builder (Algorithm 1 of
"ApproxTrain", Section V-A) agrees with the oracle's, and argument checks that
run before any HIP call return the documented status."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, pm_one

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def am():
    import approximate_multiplier_dnn_amd as m
    return m


def test_library_exports_every_declared_function(am):
    with open(os.path.join(ROOT, "include", "approx_mul.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:int|long long|const char \*)\s*(approx_\w+)\s*\(", header, re.M))
    assert declared == set(am.EXPORTS)
    lib = ctypes.CDLL(am.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_library_built_from_these_sources(am):
    """The loaded binary carries the stamp of the sources beside it (a stale
    build would not)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_approx_build", os.path.join(ROOT, "approximate_multiplier_dnn_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    assert am.approx_build_id() == b.source_hash()


@pytest.mark.parametrize("M", list(range(1, 12)))
def test_builtin_tables_match_oracle(am, M):
    for model, name in ((am.MODEL_EXACT, "exact"), (am.MODEL_MITCHELL, "mitchell")):
        assert np.array_equal(am.approx_lut_build(model, M), oracle.lut_generate(M, name))


def test_perturbed_table_matches_oracle(am):
    delta = pm_one(PERTURB_SEED, 1 << 16)
    lib_t = am.approx_lut_build(am.MODEL_EXACT, 8, delta)
    orc_t = oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), delta)
    assert np.array_equal(lib_t, orc_t)


def test_table_from_user_model(am):
    t = am.approx_lut_build_from_model(5, lambda a, b: np.float32(a) * np.float32(b))
    assert np.array_equal(t, oracle.lut_generate(5, "exact"))
    with pytest.raises(am.ApproxError) as e:
        am.approx_lut_build_from_model(4, lambda a, b: 0.25 * a * b)
    assert e.value.status == am.APPROX_EUNSUPPORTED


def test_argument_errors_before_any_device_call(am):
    L = am.lib()
    out = np.zeros(16, np.uint16)
    assert L.approx_lut_build(7, 3, None, out.ctypes.data) == am.APPROX_EINVAL       # unknown model
    assert L.approx_lut_build(0, 12, None, out.ctypes.data) == am.APPROX_EUNSUPPORTED
    assert L.approx_lut_build(0, 3, None, None) == am.APPROX_EINVAL
    assert L.approx_lut_load(None, 7) == am.APPROX_EINVAL
    assert L.approx_lut_load(out.ctypes.data, 12) == am.APPROX_EUNSUPPORTED         # M above 11
    assert L.approx_lut_load(out.ctypes.data, 0) == am.APPROX_EUNSUPPORTED
    p = 4096  # never dereferenced: the checks fail first
    assert L.approx_gemm(2, 0, 4, 4, 4, p, 4, p, 4, p, 4, None) == am.APPROX_EINVAL   # bad flag
    assert L.approx_gemm(0, 0, -1, 4, 4, p, 4, p, 4, p, 4, None) == am.APPROX_EINVAL
    assert L.approx_gemm(0, 0, 4, 4, 4, p, 3, p, 4, p, 4, None) == am.APPROX_EINVAL   # lda < k
    assert L.approx_gemm(0, 1, 4, 4, 8, p, 8, p, 7, p, 4, None) == am.APPROX_EINVAL   # ldb < k (transB)
    assert L.approx_gemm(0, 0, 4, 5, 4, p, 4, p, 5, p, 4, None) == am.APPROX_EINVAL   # ldc < n
    assert L.approx_gemm(0, 0, 4, 4, 4, None, 4, p, 4, p, 4, None) == am.APPROX_EINVAL
    assert L.approx_gemm(0, 0, 4, 4, 4, p, 4, p, 4, None, 4, None) == am.APPROX_EINVAL
    assert L.approx_gemm(0, 0, 0, 4, 4, p, 4, p, 4, p, 4, None) == am.APPROX_OK        # empty: no-op
    assert L.approx_gemm_strided_batched(0, 0, 4, 4, 4, p, 4, -1, p, 4, 0, p, 4, 16, 2, None) == am.APPROX_EINVAL
    assert L.approx_gemm_strided_batched(0, 0, 4, 4, 4, p, 4, 0, p, 4, 0, p, 4, 16, -2, None) == am.APPROX_EINVAL
    for fn in (L.approx_conv2d_fwd, L.approx_conv2d_dgrad, L.approx_conv2d_wgrad):
        assert fn(1, 4, 4, 2, 2, 3, 3, 0, 1, 1, 1, p, p, p, None) == am.APPROX_EINVAL   # stride 0
        assert fn(1, 4, 4, 2, 2, 7, 3, 1, 1, 1, 1, p, p, p, None) == am.APPROX_EINVAL   # R > H + 2 pad
        assert fn(1, 4, 4, 2, 2, 3, 3, 1, 1, -1, 1, p, p, p, None) == am.APPROX_EINVAL
        assert fn(1, 4, 4, 2, 2, 3, 3, 1, 1, 1, 1, None, p, p, None) == am.APPROX_EINVAL
    assert am.approx_status_string(am.APPROX_ENOLUT) == "no table loaded on this device"


def test_exponent_width_checked_before_any_device_call(am):
    L = am.lib()
    assert L.approx_exponent_bits_set(0) == am.APPROX_EUNSUPPORTED
    assert L.approx_exponent_bits_set(9) == am.APPROX_EUNSUPPORTED
    assert L.approx_exponent_bits_set(-3) == am.APPROX_EUNSUPPORTED


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
