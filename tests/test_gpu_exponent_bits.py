"""GPU parity of the (1, E, M) formats (exponent widths below 8 with the
exponent cast, "ApproxTrain" Section V) against the oracle: products
bit-exact (GEMMs with k = 1) through the fast path (every product inside the
format's range), the checked path and the forced checked path, for tables in
LDS and in global memory; sums within the gate for dense, row-vector and
Conv2D calls."""
import os

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one, special_values, splitmix64
from parity import gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def am():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import approximate_multiplier_dnn_amd as m
    return m


@pytest.fixture
def fmt(am):
    """Sets the exponent width for one test and restores FP32's afterwards."""
    def set_e(E):
        am.approx_exponent_bits_set(E)
        assert am.approx_exponent_bits() == E
    yield set_e
    am.approx_exponent_bits_set(8)


TABLES = {
    "exact7": lambda: (7, oracle.lut_generate(7, "exact")),
    "mitchell7": lambda: (7, oracle.lut_generate(7, "mitchell")),
    "mitchell3": lambda: (3, oracle.lut_generate(3, "mitchell")),
    "perturbed8": lambda: (8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16))),
    "mitchell9": lambda: (9, oracle.lut_generate(9, "mitchell")),
}


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def operands(seed, count, E, spread):
    """FP32 bit patterns with random signs and mantissas and exponents within
    `spread` of the format's range (spread < 0: that far inside it), plus the
    special values."""
    bias = (1 << (E - 1)) - 1
    lo, hi = max(1, 127 - bias + 1 - spread), min(254, 127 + bias + spread)
    r = splitmix64(seed, 3 * count)
    sign = (r[0::3] & np.uint64(1)).astype(np.uint32) << np.uint32(31)
    exp = (lo + (r[1::3] % np.uint64(max(1, hi - lo + 1)))).astype(np.uint32)
    frac = (r[2::3] >> np.uint64(41)).astype(np.uint32) & np.uint32(0x7FFFFF)
    return np.concatenate([sign | (exp << np.uint32(23)) | frac, special_values().view(np.uint32)])


def products(am, a, b):
    A = dev(a.view(np.float32).reshape(-1, 1))
    B = dev(b.view(np.float32).reshape(1, -1))
    C = torch.empty((a.size, b.size), dtype=torch.float32, device="cuda")
    am.approx_gemm(0, 0, a.size, b.size, 1, A, 1, B, b.size, C, b.size)
    return host(C).view(np.uint32)


def compare(got, a, b, t, M, E):
    want = oracle.amsim_bits(np.repeat(a, b.size), np.tile(b, a.size), t, M, E).reshape(a.size, b.size)
    want = np.where(want == 0x80000000, 0, want).astype(np.uint32)     # +0 + (-0) = +0
    gnan = np.isnan(got.view(np.float32))
    assert np.array_equal(gnan, np.isnan(want.view(np.float32)))
    bad = np.count_nonzero(got[~gnan] != want[~gnan])
    assert bad == 0, f"{bad} products differ"


@pytest.mark.parametrize("name", sorted(TABLES))
@pytest.mark.parametrize("E", [1, 2, 3, 5, 7])
@pytest.mark.parametrize("mode", ["across", "checked"])
def test_products_bit_exact(am, fmt, name, E, mode):
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    fmt(E)
    a = operands(900 + E, 300, E, 3)
    b = operands(901 + E, 200, E, 3)
    print(f"format products {name} E={E} {mode}", flush=True)
    if mode == "checked":
        os.environ["APPROX_FORCE_CHECKED"] = "1"
    try:
        got = products(am, a, b)
    finally:
        os.environ.pop("APPROX_FORCE_CHECKED", None)
    compare(got, a, b, t, M, E)


@pytest.mark.parametrize("name", ["exact7", "perturbed8", "mitchell9"])
def test_products_inside_the_range_take_the_fast_path(am, fmt, name):
    """E = 6 (normal 2^-30 .. 2^31) with operand exponents in -12 .. 12: no
    product leaves the range, so the fast path runs; it must give the rule's
    bits, and the same bits as the forced checked path."""
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    fmt(6)
    r = splitmix64(950, 3 * 400)
    bits = ((r[0::3] & np.uint64(1)).astype(np.uint32) << np.uint32(31)) | \
        ((115 + r[1::3] % np.uint64(25)).astype(np.uint32) << np.uint32(23)) | \
        ((r[2::3] >> np.uint64(41)).astype(np.uint32) & np.uint32(0x7FFFFF))
    a, b = bits[:240], bits[240:]
    got = products(am, a, b)
    compare(got, a, b, t, M, 6)
    os.environ["APPROX_FORCE_CHECKED"] = "1"
    try:
        got2 = products(am, a, b)
    finally:
        os.environ.pop("APPROX_FORCE_CHECKED", None)
    assert np.array_equal(got, got2)


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8"])
@pytest.mark.parametrize("E", [4, 5])
def test_gemm_and_row_vector_sums(am, fmt, name, E):
    """N(0, 1) operands scaled so that some fall outside the E-bit range."""
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    fmt(E)
    scale = 2.0 ** (1 << (E - 1)) / 16
    for (m, n, k) in ((70, 45, 130), (3, 300, 257), (1, 64, 1000)):
        A = normal(960 + m, (m, k), std=scale)
        B = normal(961 + m, (k, n), std=1.0 / scale)
        R, S = oracle.gemm(A, B, t, M, E=E)
        print(f"format gemm {name} E={E} {m}x{n}x{k}", flush=True)
        gate(host(am.gemm(dev(A), dev(B))), R, S, what=f"E={E} {m}x{n}x{k}")


def test_conv(am, fmt):
    M, t = TABLES["mitchell7"]()
    am.approx_lut_load(t, M)
    fmt(4)
    N, H, W, C, K, R, S, stride, pad = (2, 7, 9, 5, 6, 3, 3, (1, 1), (1, 1))
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(971, (N, H, W, C), std=8.0)
    w = normal(972, (R, S, C, K), std=0.5)
    dy = normal(973, (N, P, Q, K), std=4.0)
    Y, YS = oracle.conv2d_fwd(x, w, t, M, stride, pad, E=4)
    gate(host(am.conv2d_fwd(dev(x), dev(w), stride, pad)), Y, YS, what="fwd")
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, t, M, stride, pad, E=4)
    gate(host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, stride, pad)), DX, DXS, what="dgrad")
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, t, M, stride, pad, E=4)
    gate(host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, stride, pad)), DW, DWS, what="wgrad")


def test_width_persists_and_native_ignores_it(am, fmt):
    M, t = TABLES["exact7"]()
    fmt(3)
    am.approx_lut_load(t, M)                  # a table load keeps the width
    assert am.approx_exponent_bits() == 3
    am.approx_native_load()                   # the native multiplier is FP32 throughout
    A = np.array([[1000.0, 2.0 ** -20]], np.float32)
    B = np.array([[1000.0], [3.0]], np.float32)
    got = host(am.gemm(dev(A), dev(B)))
    assert got[0, 0] == np.float32(1000.0 * 1000.0 + 3 * 2.0 ** -20)
    am.approx_lut_load(t, M)


@pytest.mark.parametrize("name", ["exact7", "mitchell3", "perturbed8", "mitchell9"])
@pytest.mark.parametrize("E", [2, 3, 5, 8])
def test_products_with_underflow_take_the_ranged_path(am, fmt, name, E):
    """Operand exponents from 3 below the format's range up to the middle of
    it: products can fall below the range but not above it (the fast path
    with underflow). Bit-exact against the oracle and the forced checked
    path; E = 8 covers FP32's own underflow."""
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    fmt(E)
    bias = (1 << (E - 1)) - 1
    lo, hi = max(1, 128 - bias - 3), 127 + bias // 2
    r = splitmix64(990 + E, 3 * 500)
    bits = ((r[0::3] & np.uint64(1)).astype(np.uint32) << np.uint32(31)) | \
        ((lo + r[1::3] % np.uint64(hi - lo + 1)).astype(np.uint32) << np.uint32(23)) | \
        ((r[2::3] >> np.uint64(41)).astype(np.uint32) & np.uint32(0x7FFFFF))
    zeros_nan = np.array([0x00000000, 0x80000000, 0x7FC00000, 0x00000001], np.uint32)
    a = np.concatenate([bits[:280], zeros_nan])
    b = np.concatenate([bits[280:], zeros_nan])
    print(f"ranged products {name} E={E}", flush=True)
    got = products(am, a, b)
    compare(got, a, b, t, M, E)
    os.environ["APPROX_FORCE_CHECKED"] = "1"
    try:
        got2 = products(am, a, b)
    finally:
        os.environ.pop("APPROX_FORCE_CHECKED", None)
    gnan = np.isnan(got.view(np.float32))
    assert np.array_equal(gnan, np.isnan(got2.view(np.float32)))
    assert np.array_equal(got[~gnan], got2[~gnan])
