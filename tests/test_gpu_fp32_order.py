"""GPU results bit for bit against the oracle's FP32 sums in the documented
order (reading R20), with each output's chunk length taken from the library
(approx_gemm_chunks, approx_conv2d_chunks).

This is where FP32 accumulation itself is checked, including what a double
sum cannot show: partial sums that overflow to infinity part-way, an infinity
met by one of the other sign (NaN), cancellations whose result depends on the
order. Products of large finite operands go through the checked path (a
product may overflow) and through the fast path (every product stays finite
while the sums overflow). Every kernel route is covered: whole tiles, tiles
split into chunks, only the last round's tiles split, the row-vector kernel
with and without a split, batches by stride and by pointer array, tables in
LDS and in global memory, the native multiplier, and the three Conv2D passes.
"""
import os

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one, splitmix64
from parity import gate, same_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

_T = {}


def table(name):
    if name not in _T:
        if name == "mitchell7":
            _T[name] = (7, oracle.lut_generate(7, "mitchell"))
        elif name == "exact7":
            _T[name] = (7, oracle.lut_generate(7, "exact"))
        elif name == "perturbed8":
            _T[name] = (8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16)))
        elif name == "arbitrary10":
            _T[name] = (10, (splitmix64(7010, 1 << 20) >> np.uint64(48)).astype(np.uint16))
        else:
            _T[name] = (0, None)
    return _T[name]


@pytest.fixture(scope="module")
def am():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import approximate_multiplier_dnn_amd as m
    yield m
    m.approx_exponent_bits_set(8)
    m.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)


def use(am, name):
    M, t = table(name)
    if t is None:
        am.approx_native_load()
    else:
        am.approx_lut_load(t, M)
    return M, t


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(x):
    torch.cuda.synchronize()
    return x.cpu().numpy()


def check_gemm(am, name, A, B, C, transA=False, transB=False, what=""):
    """Every output of C against the FP32-order oracle, bit for bit."""
    M, t = table(name)
    m, n = C.shape
    k = A.shape[0] if transA else A.shape[1]
    rows, cols = np.meshgrid(np.arange(m, dtype=np.int32), np.arange(n, dtype=np.int32), indexing="ij")
    rows, cols = rows.ravel(), cols.ravel()
    L = am.approx_gemm_chunks(int(transA), int(transB), m, n, k, 1, 0, rows, cols)
    F = oracle.gemm_f32_at(A, B, t, M, rows, cols, np.maximum(L, 1), transA=transA, transB=transB,
                           threads=oracle.default_threads())
    same_bits(C, F, what=what, zero_sign=t is not None)
    return L


# (m, n, k, route the plan takes)
ROUTES = [
    ((2048, 4096, 128), "GEMM kernel, whole tiles"),     # 256 tiles: one full round
    ((96, 80, 3000), "GEMM kernel, every tile split"),
    ((300, 40, 9000), "GEMM kernel, long split"),
    ((8, 3000, 2500), "row-vector kernel, split"),
    ((1, 200, 12), "row-vector kernel, one chunk"),
    ((40, 1000, 5000), "row-vector kernel, 10 row blocks"),
]


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8", "arbitrary10", "native"])
@pytest.mark.parametrize("shape,route", ROUTES, ids=[r[1] for r in ROUTES])
def test_routes_bit_exact(am, name, shape, route):
    M, t = use(am, name)
    m, n, k = shape
    print(f"fp32 order {name} {shape} {route}", flush=True)
    A = normal(1500 + m, (m, k))
    B = normal(1501 + n, (k, n))
    C = host(am.gemm(dev(A), dev(B)))
    L = check_gemm(am, name, A, B, C, what=f"{name} {shape}")
    if "split" in route:
        assert np.any(L < k), f"{route}: expected a split plan, chunks {np.unique(L)}"
    elif "whole" in route or "one chunk" in route:
        assert np.all(L == k), f"{route}: expected one chunk per output, chunks {np.unique(L)}"


def test_tail_tiles_split_bit_exact(am):
    """260 row tiles of 512 rows x 64 columns: one full round of whole tiles
    and the 4 tiles of the last round split, whose chunk partials are summed
    by the tile reduction; the chunk length differs between the two kinds."""
    use(am, "mitchell7")
    m, n, k = 260 * 512 - 100, 64, 400
    A = normal(1510, (m, k))
    B = normal(1511, (k, n))
    C = host(am.gemm(dev(A), dev(B)))
    L = check_gemm(am, "mitchell7", A, B, C, what="tail tiles")
    if not os.environ.get("APPROX_KERNEL_SHAPE"):    # the tiling described above is the default shape's
        assert np.any(L == k) and np.any(L < k), np.unique(L)


@pytest.mark.parametrize("transA,transB", [(0, 1), (1, 0), (1, 1)])
def test_transposes_bit_exact(am, transA, transB):
    use(am, "perturbed8")
    m, n, k = 330, 150, 700
    A = normal(1520 + transA, (k, m) if transA else (m, k))
    B = normal(1521 + transB, (n, k) if transB else (k, n))
    C = host(am.gemm(dev(A), dev(B), transA=bool(transA), transB=bool(transB)))
    check_gemm(am, "perturbed8", A, B, C, bool(transA), bool(transB), what=f"trans {transA}{transB}")


def test_batched_pointer_arrays_bit_exact(am):
    """Attention-like products through a pointer array: each entry's outputs
    follow the order reported for its batch index."""
    M, t = use(am, "mitchell7")
    nb, T, dh = 6, 200, 64
    Q = [normal(1530 + i, (T, dh)) for i in range(nb)]
    K = [normal(1540 + i, (T, dh)) for i in range(nb)]
    dQ, dK = [dev(q) for q in Q], [dev(x) for x in K]
    S = [torch.empty((T, T), dtype=torch.float32, device="cuda") for _ in range(nb)]
    am.approx_gemm_batched(0, 1, T, T, dh, am.pointer_array(dQ), dh, am.pointer_array(dK), dh,
                           am.pointer_array(S), T, nb)
    torch.cuda.synchronize()
    rows, cols = np.meshgrid(np.arange(T, dtype=np.int32), np.arange(T, dtype=np.int32), indexing="ij")
    for b in range(nb):
        L = am.approx_gemm_chunks(0, 1, T, T, dh, nb, b, rows.ravel(), cols.ravel())
        F = oracle.gemm_f32_at(Q[b], K[b], t, M, rows.ravel(), cols.ravel(), np.maximum(L, 1), transB=True)
        same_bits(S[b].cpu().numpy(), F, what=f"pointer batch {b}")


# ---------------------------------------------------------------- overflow

X = np.float32(1.5 * 2.0 ** 127)


def big_operands(seed, m, n, k, scale, density):
    """N(0, 1) operands; about `density` of A's entries replaced by +-scale
    (a power of two times 1.5), so that some sums of products exceed the FP32
    maximum part-way; a few infinities in B."""
    A = normal(seed, (m, k))
    B = normal(seed + 1, (k, n))
    r = splitmix64(seed + 2, m * k)
    hit = (r % np.uint64(1000000)) < np.uint64(int(1000000 * density))
    sign = np.where((r >> np.uint64(40)) & np.uint64(1), -1.0, 1.0).astype(np.float32)
    flatA = A.reshape(-1)
    flatA[hit] = sign[hit] * np.float32(scale)
    rb = splitmix64(seed + 3, k * n)
    infs = (rb % np.uint64(5000)) == np.uint64(0)
    flatB = B.reshape(-1)
    flatB[infs] = np.where((rb[infs] >> np.uint64(30)) & np.uint64(1), np.inf, -np.inf).astype(np.float32)
    return A, B


@pytest.mark.parametrize("name", ["exact7", "perturbed8"])
@pytest.mark.parametrize("shape", [(300, 120, 400), (6, 700, 900), (64, 48, 6000)])
@pytest.mark.parametrize("scale", ["checked", "fast"])
def test_accumulator_overflow_bit_exact(am, name, shape, scale):
    """Sums that overflow to +-Inf part-way and meet infinities of the other
    sign. scale 'checked': operands of 1.5 * 2^127 (a product could exceed
    the range, so the checked path runs); 'fast': 1.5 * 2^125 against |B| < 4
    (every product stays finite: the fast path; the sums still overflow)."""
    M, t = use(am, name)
    m, n, k = shape
    s = float(X) if scale == "checked" else 1.5 * 2.0 ** 125
    A, B = big_operands(1550 + m + k, m, n, k, s, (2.0 if scale == "checked" else 6.0) / k)
    if scale == "fast":
        B = np.where(np.isinf(B), B, np.clip(B, -3.99, 3.99)).astype(np.float32)
    C = host(am.gemm(dev(A), dev(B)))
    with np.errstate(over="ignore", invalid="ignore"):
        F_inf = np.isinf(C).sum()
    print(f"overflow {name} {shape} {scale}: {F_inf} infinite, {np.isnan(C).sum()} NaN outputs", flush=True)
    check_gemm(am, name, A, B, C, what=f"overflow {name} {shape} {scale}")
    assert np.isinf(C).any() or np.isnan(C).any(), "the case should overflow somewhere"


def test_overflow_order_decides(am):
    """X + X - X overflows, X - X + X does not: the library's order, not a
    rearrangement, decides (one output each, k = 3, one chunk)."""
    use(am, "exact7")
    A = np.array([[X, X, -X], [X, -X, X]], np.float32)
    B = np.ones((3, 1), np.float32)
    C = host(am.gemm(dev(A), dev(B)))
    assert np.isinf(C[0, 0]) and C[0, 0] > 0
    assert C[1, 0] == X


# ---------------------------------------------------------------- Conv2D

CONV_GEOMS = [
    # N, H, W, C, K, R, S, stride, pad
    (4, 16, 16, 8, 12, 3, 3, (1, 1), (1, 1)),
    (2, 13, 11, 5, 7, 3, 2, (2, 1), (1, 0)),
    (3, 9, 9, 16, 3, 5, 5, (2, 2), (2, 2)),
    (20, 12, 12, 6, 10, 3, 3, (1, 1), (1, 1)),
]


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8", "native"])
@pytest.mark.parametrize("geom", CONV_GEOMS)
def test_conv_passes_bit_exact(am, name, geom):
    M, t = use(am, name)
    N, H, W, C, K, R, S, st, pd = geom
    P, Q = oracle.conv_out_hw(H, W, R, S, st, pd)
    x = normal(1600 + H, (N, H, W, C))
    w = normal(1601 + C, (R, S, C, K), std=0.2)
    dy = normal(1602 + K, (N, P, Q, K))
    outs = {"fwd": (host(am.conv2d_fwd(dev(x), dev(w), st, pd)), x, w),
            "dgrad": (host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, st, pd)), dy, w),
            "wgrad": (host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, st, pd)), x, dy)}
    for pname, (got, t1, t2) in outs.items():
        idx = np.arange(got.size, dtype=np.int64)
        L = am.approx_conv2d_chunks(pname, N, H, W, C, K, R, S, st, pd, idx)
        F = oracle.conv2d_f32(pname, t1, t2, geom, t, M, L, idx=idx, threads=oracle.default_threads())
        same_bits(got, F, what=f"conv {name} {geom} {pname}", zero_sign=t is not None)


def test_chunk_query_argument_errors(am):
    use(am, "mitchell7")
    L = am.lib()
    one = np.zeros(1, np.int32)
    out = np.zeros(1, np.int64)
    p = one.ctypes.data
    assert L.approx_gemm_chunks(0, 0, 4, 4, 4, 1, 1, p, p, p, out.ctypes.data) == am.APPROX_OK
    assert L.approx_gemm_chunks(2, 0, 4, 4, 4, 1, 1, p, p, p, out.ctypes.data) == am.APPROX_EINVAL
    bad = np.array([4], np.int32)
    assert L.approx_gemm_chunks(0, 0, 4, 4, 4, 1, 1, p, bad.ctypes.data, p, out.ctypes.data) == am.APPROX_EINVAL
    assert L.approx_gemm_chunks(0, 0, 4, 4, 4, 1, 1, None, p, p, out.ctypes.data) == am.APPROX_EINVAL
    idx = np.array([10 ** 6], np.int64)
    assert L.approx_conv2d_chunks(0, 1, 4, 4, 2, 2, 3, 3, 1, 1, 1, 1, 1, idx.ctypes.data,
                                  out.ctypes.data) == am.APPROX_EINVAL
    assert L.approx_conv2d_chunks(3, 1, 4, 4, 2, 2, 3, 3, 1, 1, 1, 1, 0, None, None) == am.APPROX_EINVAL
