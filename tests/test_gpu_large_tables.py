"""GPU parity for tables of M = 9..11 ("ApproxTrain", arXiv 2209.04161,
Section V: the mantissa width can be chosen from 1 to 11 bits). These tables
(512 KB to 8 MB) do not fit in LDS; the library reads them from global
memory. Expected values come from the oracle only: products bit-exact,
sums within the gate of tests/parity.py.

Besides the Mitchell table, an arbitrary table (every entry a seeded random
16-bit word: random carry, random mantissa) checks that the index order and
the column layout of the large image are right for any table.
"""
import os

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
    yield m
    m.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


_TABLES = {}


def table(kind, M):
    key = (kind, M)
    if key not in _TABLES:
        if kind == "mitchell":
            _TABLES[key] = oracle.lut_generate(M, "mitchell")
        else:                                   # arbitrary 16-bit entries
            _TABLES[key] = (splitmix64(7000 + M, 1 << (2 * M)) >> np.uint64(48)).astype(np.uint16)
    return _TABLES[key]


def operands(seed, M, count):
    """count normals with random mantissas at moderate exponents, both signs,
    followed by the special values."""
    r = splitmix64(seed, count)
    mant = (r & np.uint64(0x7FFFFF)).astype(np.uint32)
    exp = np.array([100, 127, 150], np.uint32)[(r >> np.uint64(32)) % np.uint64(3)]
    sign = ((r >> np.uint64(40)) & np.uint64(1)).astype(np.uint32)
    bits = (sign << np.uint32(31)) | (exp.astype(np.uint32) << np.uint32(23)) | mant
    return np.concatenate([bits, special_values().view(np.uint32)]).astype(np.uint32)


@pytest.mark.parametrize("M", [9, 10, 11])
@pytest.mark.parametrize("kind", ["mitchell", "arbitrary"])
@pytest.mark.parametrize("checked", [False, True])
def test_large_table_products_bit_exact(am, M, kind, checked):
    t = table(kind, M)
    am.approx_lut_load(t, M)
    assert am.approx_lut_bits() == M
    a = operands(100 + M, M, 360)
    b = operands(200 + M, M, 330)
    C = torch.empty((a.size, b.size), dtype=torch.float32, device="cuda")
    print(f"large-table products M={M} {kind} checked={checked}", flush=True)
    if checked:
        os.environ["APPROX_FORCE_CHECKED"] = "1"
    try:
        am.approx_gemm(0, 0, a.size, b.size, 1, dev(a.view(np.float32).reshape(-1, 1)), 1,
                       dev(b.view(np.float32).reshape(1, -1)), b.size, C, b.size)
        got = host(C).view(np.uint32)
    finally:
        os.environ.pop("APPROX_FORCE_CHECKED", None)
    want = oracle.amsim_bits(np.repeat(a, b.size), np.tile(b, a.size), t, M).reshape(a.size, b.size)
    want = np.where(want == 0x80000000, 0, want).astype(np.uint32)     # +0 + (-0) = +0
    gnan = np.isnan(got.view(np.float32))
    assert np.array_equal(gnan, np.isnan(want.view(np.float32)))
    assert np.count_nonzero(got[~gnan] != want[~gnan]) == 0


@pytest.mark.parametrize("M,kind", [(9, "arbitrary"), (11, "mitchell")])
@pytest.mark.parametrize("transA,transB", [(0, 0), (1, 1)])
@pytest.mark.parametrize("shape", [(65, 17, 129), (513, 130, 257)])
def test_large_table_gemm_parity(am, M, kind, transA, transB, shape):
    t = table(kind, M)
    am.approx_lut_load(t, M)
    m, n, k = shape
    A = normal(300 + m + transA, (k, m) if transA else (m, k))
    B = normal(400 + n + transB, (n, k) if transB else (k, n))
    R, S = oracle.gemm(A, B, t, M, transA=bool(transA), transB=bool(transB))
    C = am.gemm(dev(A), dev(B), transA=bool(transA), transB=bool(transB))
    gate(host(C), R, S, what=f"M={M} {kind} gemm {shape}")


def test_large_table_conv_parity(am):
    M = 10
    t = table("mitchell", M)
    am.approx_lut_load(t, M)
    N, H, W, C, K, R, S, stride, pad = 2, 12, 12, 16, 24, 3, 3, (1, 1), (1, 1)
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(501, (N, H, W, C))
    w = normal(502, (R, S, C, K))
    dy = normal(503, (N, P, Q, K))
    Y, YS = oracle.conv2d_fwd(x, w, t, M, stride, pad)
    gate(host(am.conv2d_fwd(dev(x), dev(w), stride, pad)), Y, YS, what="M=10 fwd")
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, t, M, stride, pad)
    gate(host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, stride, pad)), DX, DXS, what="M=10 dgrad")
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, t, M, stride, pad)
    gate(host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, stride, pad)), DW, DWS, what="M=10 wgrad")
