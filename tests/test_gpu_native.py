"""GPU parity of the native multiplier ("ApproxTrain", arXiv 2209.04161,
Section V: the simulator can call the hardware multiplication instead of the
table; Fig. 6 compares the two). With approx_native_load() selected, every
GEMM and Conv2D call must match the oracle's native sums (exact products,
float64 accumulation) within the gate of tests/parity.py, and single
products (k = 1) must equal the exact product rounded once to FP32.
"""
import numpy as np
import pytest

import oracle
from datagen import normal, special_values, splitmix64
from parity import gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def am():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import approximate_multiplier_dnn_amd as m
    m.approx_native_load()
    yield m
    m.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def test_native_is_selected(am):
    am.approx_native_load()
    assert am.approx_lut_bits() == 0


def test_native_products_are_rounded_once(am):
    """k = 1: c = fma(a, b, +0) = the exact product rounded to FP32
    (subnormal results included; zeros compare by value)."""
    am.approx_native_load()
    exps = np.array([1, 2, 40, 100, 127, 150, 200, 253, 254], np.uint32)
    mant = splitmix64(901, 24).astype(np.uint32) & np.uint32(0x7FFFFF)
    vals = [(np.uint32(s) << np.uint32(31)) | (e << np.uint32(23)) | m for e in exps for s in (0, 1) for m in mant[:3]]
    sub = np.array([1, 2, 0x3FFFFF, 0x400000, 0x7FFFFF], np.uint32)        # subnormal operands
    a = np.concatenate([np.array(vals, np.uint32), sub, special_values().view(np.uint32)]).view(np.float32)
    b = a[::-1].copy()
    C = torch.empty((a.size, b.size), dtype=torch.float32, device="cuda")
    print(f"native products {a.size} x {b.size}", flush=True)
    am.approx_gemm(0, 0, a.size, b.size, 1, dev(a.reshape(-1, 1)), 1, dev(b.reshape(1, -1)), b.size, C, b.size)
    got = host(C)
    with np.errstate(over="ignore", invalid="ignore"):
        exact = oracle.mul_native(np.repeat(a, b.size), np.tile(b, a.size))
        want = exact.astype(np.float32).reshape(a.size, b.size)
    # an exact zero product added to +0 gives +0; a non-zero product that
    # rounds to zero keeps its sign
    want = np.where(exact.reshape(a.size, b.size) == 0, np.float32(0), want)
    gnan, wnan = np.isnan(got), np.isnan(want)
    assert np.array_equal(gnan, wnan)
    # zeros compare by value: the hardware FMA returns +0 where a tiny
    # negative product rounds to zero (IEEE-754 would keep the sign); the
    # sign of a zero cannot change any sum
    both_zero = (got == 0) & (want == 0)
    bad = np.argwhere((got.view(np.uint32) != want.view(np.uint32)) & ~gnan & ~both_zero)
    for i, j in bad[:24]:
        print(f"a={a[i]!r} ({a.view(np.uint32)[i]:08x}) b={b[j]!r} ({b.view(np.uint32)[j]:08x}) "
              f"got {got[i, j]!r} ({got.view(np.uint32)[i, j]:08x}) want {want[i, j]!r} "
              f"({want.view(np.uint32)[i, j]:08x})")
    assert bad.shape[0] == 0, f"{bad.shape[0]} products differ"


@pytest.mark.parametrize("transA,transB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("shape", [(7, 5, 3), (65, 17, 129), (513, 130, 257), (20, 300, 1000)])
def test_native_gemm_parity(am, shape, transA, transB):
    am.approx_native_load()
    m, n, k = shape
    seed = 3 * m + 5 * n + k + 100 * transA + 200 * transB
    A = normal(seed, (k, m) if transA else (m, k))
    B = normal(seed + 1, (n, k) if transB else (k, n))
    R, S = oracle.gemm(A, B, None, 0, transA=bool(transA), transB=bool(transB))
    C = am.gemm(dev(A), dev(B), transA=bool(transA), transB=bool(transB))
    gate(host(C), R, S, what=f"native gemm {shape} {transA}{transB}")


def test_native_gemm_special_values(am):
    am.approx_native_load()
    A = normal(931, (40, 24))
    B = normal(932, (24, 30))
    A[3, 5] = np.inf
    A[7, :] = 0.0
    A[7, 2] = np.inf                  # Inf facing a zero of B below gives NaN
    B[2, 4] = 0.0
    B[9, 11] = np.nan
    A[11, 6] = np.float32(1.0e-41)    # subnormal operand, kept
    R, S = oracle.gemm(A, B, None, 0)
    with np.errstate(invalid="ignore"):
        gate(host(am.gemm(dev(A), dev(B))), R, S, what="native specials")


@pytest.mark.parametrize("geom", [
    (2, 8, 8, 4, 5, 3, 3, (1, 1), (1, 1)),
    (1, 9, 7, 3, 2, 3, 3, (2, 2), (1, 1)),
    (2, 6, 10, 5, 3, 3, 2, (2, 1), (0, 1)),
    (1, 10, 9, 2, 2, 4, 3, (3, 2), (1, 0)),
    (2, 16, 16, 64, 64, 3, 3, (1, 1), (1, 1)),
])
def test_native_conv_parity(am, geom):
    am.approx_native_load()
    N, H, W, C, K, R, S, stride, pad = geom
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(941, (N, H, W, C))
    w = normal(942, (R, S, C, K))
    dy = normal(943, (N, P, Q, K))
    print(f"native conv {geom}", flush=True)
    Y, YS = oracle.conv2d_fwd(x, w, None, 0, stride, pad)
    gate(host(am.conv2d_fwd(dev(x), dev(w), stride, pad)), Y, YS, what="native fwd")
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, None, 0, stride, pad)
    gate(host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, stride, pad)), DX, DXS, what="native dgrad")
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, None, 0, stride, pad)
    gate(host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, stride, pad)), DW, DWS, what="native wgrad")


def test_native_gemm8192_sampled(am):
    """The 8192^3 GEMM in the launch configuration the benchmark's native
    comparison times, on sampled outputs."""
    from datagen import configs as cfg
    am.approx_native_load()
    A, B = cfg.gemm_square(4, 8192)
    print("native gemm 8192^3", flush=True)
    C = host(am.gemm(dev(A), dev(B)))
    r = splitmix64(951, 2 * 2048)
    rows = (r[0::2] % np.uint64(A.shape[0])).astype(np.int32)
    cols = (r[1::2] % np.uint64(B.shape[1])).astype(np.int32)
    R, S = oracle.gemm_at(A, B, None, 0, rows, cols)
    gate(C[rows, cols], R, S, what="native 8192")


def test_table_selected_again_after_native(am):
    am.approx_native_load()
    A = normal(961, (33, 20))
    B = normal(962, (20, 9))
    t = oracle.lut_generate(7, "mitchell")
    am.approx_lut_load(t, 7)
    assert am.approx_lut_bits() == 7
    R, S = oracle.gemm(A, B, t, 7)
    gate(host(am.gemm(dev(A), dev(B))), R, S, what="table after native")
