"""GPU parity of the row-vector path: approx_gemm with at most 32 rows in
op(A) (64 when k * n >= 2^22 or k * n <= 2^16), in blocks of 4 rows, and B not
transposed (batch-1 and few-row dense inference; ApproxTrain,
arXiv 2209.04161, Section VI-D, keeps a separate matrix-vector kernel for
this case). The library routes these calls to a kernel whose lanes run over
the output columns; products must equal the oracle's bit for bit (k = 1) and
sums pass the gate of tests/parity.py, for tables in LDS range and beyond it,
and for the native multiplier.
"""
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
    yield m
    m.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


_T = {}


def use(am, name):
    """Load a table (or the native multiplier); returns (table or None, M)."""
    if name not in _T:
        if name == "mitchell7":
            _T[name] = (oracle.lut_generate(7, "mitchell"), 7)
        elif name == "exact7":
            _T[name] = (oracle.lut_generate(7, "exact"), 7)
        elif name == "perturbed8":
            _T[name] = (oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16)), 8)
        elif name == "arbitrary11":
            _T[name] = ((splitmix64(7011, 1 << 22) >> np.uint64(48)).astype(np.uint16), 11)
        elif name.startswith("arbitrary"):      # arbitrary 16-bit entries, M = 1..8
            M = int(name[len("arbitrary"):])
            _T[name] = ((splitmix64(7100 + M, 1 << (2 * M)) >> np.uint64(48)).astype(np.uint16), M)
        else:
            _T[name] = (None, 0)
    t, M = _T[name]
    if t is None:
        am.approx_native_load()
    else:
        am.approx_lut_load(t, M)
    return t, M


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8", "arbitrary11", "native"])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 13, 16])
@pytest.mark.parametrize("transA", [0, 1])
# the per-item index counts (chunks) these shapes give cover every residue
# of the kernel's groups of 4 and 8 indices: 1, 7, 9, 8, 12, 16 and 10 among them
@pytest.mark.parametrize("nk", [(1, 1), (5, 7), (1000, 300), (1025, 2049), (4096, 513), (2050, 2048),
                                (600, 3072), (300, 4096), (700, 2560)])
def test_gemv_parity(am, name, m, transA, nk):
    n, k = nk
    t, M = use(am, name)
    seed = 11 * m + 7 * n + k + 50 * transA
    A = normal(seed, (k, m) if transA else (m, k))
    B = normal(seed + 1, (k, n))
    R, S = oracle.gemm(A, B, t, M, transA=bool(transA))
    C = am.gemm(dev(A), dev(B), transA=bool(transA))
    gate(host(C), R, S, what=f"gemv {name} m={m} {nk} tA={transA}")


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8", "arbitrary11"])
def test_gemv_products_bit_exact(am, name):
    """k = 1: every output is +0 + one approximate product."""
    t, M = use(am, name)
    r = splitmix64(900 + M, 900)
    mant = (r & np.uint64(0x7FFFFF)).astype(np.uint32)
    exp = np.array([1, 60, 127, 190, 254], np.uint32)[(r >> np.uint64(32)) % np.uint64(5)]
    sign = ((r >> np.uint64(40)) & np.uint64(1)).astype(np.uint32)
    bvals = np.concatenate([(sign << np.uint32(31)) | (exp << np.uint32(23)) | mant,
                            special_values().view(np.uint32)]).astype(np.uint32)
    avals = np.concatenate([bvals[:2], special_values().view(np.uint32)[:2]]).astype(np.uint32)  # m = 4 rows
    C = torch.empty((4, bvals.size), dtype=torch.float32, device="cuda")
    am.approx_gemm(0, 0, 4, bvals.size, 1, dev(avals.view(np.float32).reshape(4, 1)), 1,
                   dev(bvals.view(np.float32).reshape(1, -1)), bvals.size, C, bvals.size)
    got = host(C).view(np.uint32)
    want = oracle.amsim_bits(np.repeat(avals, bvals.size), np.tile(bvals, 4), t, M).reshape(4, bvals.size)
    want = np.where(want == 0x80000000, 0, want).astype(np.uint32)
    gnan = np.isnan(got.view(np.float32))
    assert np.array_equal(gnan, np.isnan(want.view(np.float32)))
    assert np.count_nonzero(got[~gnan] != want[~gnan]) == 0


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8", "arbitrary11"])
def test_gemv_special_b_on_the_fast_path(am, name):
    """k = 1 with op(A) and B of moderate exponents (no product can leave the
    range) and B holding +-0, subnormals, +-Inf and NaN: every product bit for
    bit. Zeros and subnormals keep a wave on the fast path; an Inf or NaN B
    sends its wave to the checked path."""
    t, M = use(am, name)
    r = splitmix64(950 + M, 700)
    mant = (r & np.uint64(0x7FFFFF)).astype(np.uint32)
    exp = (100 + (r >> np.uint64(32)) % np.uint64(50)).astype(np.uint32)
    sign = ((r >> np.uint64(40)) & np.uint64(1)).astype(np.uint32)
    bvals = ((sign << np.uint32(31)) | (exp << np.uint32(23)) | mant).astype(np.uint32)
    spec = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x7F800000, 0xFF800000,
                     0x7FC00000, 0xFFC00001, 0x7F800001], np.uint32)
    bvals[3::61] = spec[np.arange(bvals[3::61].size) % spec.size]
    avals = np.array([0x3FC00000, 0xC1234567, 0x00000000, 0x7F800000], np.uint32)   # 1.5, -10.2, 0, Inf
    C = torch.empty((4, bvals.size), dtype=torch.float32, device="cuda")
    am.approx_gemm(0, 0, 4, bvals.size, 1, dev(avals.view(np.float32).reshape(4, 1)), 1,
                   dev(bvals.view(np.float32).reshape(1, -1)), bvals.size, C, bvals.size)
    got = host(C).view(np.uint32)
    want = oracle.amsim_bits(np.repeat(avals, bvals.size), np.tile(bvals, 4), t, M).reshape(4, bvals.size)
    want = np.where(want == 0x80000000, 0, want).astype(np.uint32)     # +0 + (-0) = +0
    gnan = np.isnan(got.view(np.float32))
    assert np.array_equal(gnan, np.isnan(want.view(np.float32)))
    assert np.count_nonzero(got[~gnan] != want[~gnan]) == 0


@pytest.mark.parametrize("name,m,n,k", [("exact7", 64, 64, 64), ("perturbed8", 48, 8192, 1024),
                                        ("perturbed8", 1, 8192, 4096), ("mitchell7", 1, 2050, 2048),
                                        ("mitchell7", 5, 3000, 700), ("arbitrary11", 3, 2000, 900)])
def test_gemv_fast_and_forced_checked_agree_bitwise(am, name, m, n, k):
    """The row-vector kernels' fast path (and the one-row kernel's per-window
    test) against the same call forced onto the per-product checked path:
    every output bit for bit. N(0, 1) operands, on which every wave takes the
    fast path unless forced: 64 x 64 x 64 (the smallest bench workload), 48
    rows with k * n >= 2^22, the one-row kernel, and the table in global
    memory."""
    use(am, name)
    A = dev(normal(9870 + m, (m, k)))
    B = dev(normal(9871 + m, (k, n)))
    outs = []
    for forced in (False, True):
        C = torch.full((m, n), -5.0, dtype=torch.float32, device="cuda")
        if forced:
            os.environ["APPROX_FORCE_CHECKED"] = "1"
        try:
            am.approx_gemm(0, 0, m, n, k, A, k, B, n, C, n)
            outs.append(host(C).view(np.uint32).copy())
        finally:
            os.environ.pop("APPROX_FORCE_CHECKED", None)
    assert np.isfinite(outs[0].view(np.float32)).all()
    assert np.count_nonzero(outs[0] != outs[1]) == 0, f"{name} {m}x{n}x{k}: fast and checked differ"


@pytest.mark.parametrize("name", ["arbitrary1", "arbitrary2", "arbitrary3", "arbitrary5", "arbitrary8"])
def test_gemv_small_tables_bit_exact(am, name):
    """Tables of M = 1..8 with arbitrary entries, staged in LDS as padded rows
    (rows of 2 and 4 entries copied one entry at a time, wider rows 16 bytes
    at a time): k = 1 products bit for bit, specials included, then a
    row-vector sum."""
    t, M = use(am, name)
    r = splitmix64(960 + M, 600)
    mant = (r & np.uint64(0x7FFFFF)).astype(np.uint32)
    exp = (110 + (r >> np.uint64(32)) % np.uint64(30)).astype(np.uint32)
    sign = ((r >> np.uint64(40)) & np.uint64(1)).astype(np.uint32)
    bvals = ((sign << np.uint32(31)) | (exp << np.uint32(23)) | mant).astype(np.uint32)
    bvals[5::47] = special_values().view(np.uint32)[[0, 1, 2, 19, 20, 21, 22, 23, 0, 1, 2, 19, 20]][:bvals[5::47].size]
    avals = np.concatenate([bvals[100:103], np.array([0x7FC00000], np.uint32)])
    C = torch.empty((4, bvals.size), dtype=torch.float32, device="cuda")
    am.approx_gemm(0, 0, 4, bvals.size, 1, dev(avals.view(np.float32).reshape(4, 1)), 1,
                   dev(bvals.view(np.float32).reshape(1, -1)), bvals.size, C, bvals.size)
    got = host(C).view(np.uint32)
    want = oracle.amsim_bits(np.repeat(avals, bvals.size), np.tile(bvals, 4), t, M).reshape(4, bvals.size)
    want = np.where(want == 0x80000000, 0, want).astype(np.uint32)
    gnan = np.isnan(got.view(np.float32))
    assert np.array_equal(gnan, np.isnan(want.view(np.float32)))
    assert np.count_nonzero(got[~gnan] != want[~gnan]) == 0
    A = normal(970 + M, (2, 700))
    B = normal(971 + M, (700, 900))
    R, S = oracle.gemm(A, B, t, M)
    gate(host(am.gemm(dev(A), dev(B))), R, S, what=f"gemv {name}")


@pytest.mark.parametrize("m", [6, 16])
def test_gemv_row_blocks_strided_batch_and_padding(am, m):
    """More than 4 rows run as blocks of 4 rows in the row-vector kernel: a strided
    batch with padded leading dimensions, op(A) transposed or not; the
    padding of C is not written."""
    t, M = use(am, "perturbed8")
    n, k, batch = 2100, 2000, 2
    for transA in (0, 1):
        lda = (m if transA else k) + 5
        ar = k if transA else m
        A = normal(990 + m + transA, (batch, ar, lda))
        B = normal(991 + m, (batch, k, n + 2))
        C = torch.full((batch, m, n + 4), 5.0, dtype=torch.float32, device="cuda")
        am.approx_gemm_strided_batched(transA, 0, m, n, k, dev(A), lda, ar * lda, dev(B), n + 2, k * (n + 2),
                                       C, n + 4, m * (n + 4), batch)
        got = host(C)
        for b in range(batch):
            Ab = A[b][:, :m] if transA else A[b][:, :k]
            R, S = oracle.gemm(Ab, B[b][:, :n], t, M, transA=bool(transA))
            gate(got[b][:, :n], R, S, what=f"row blocks m={m} tA={transA} b={b}")
        assert np.all(got[:, :, n:] == 5.0)


def test_gemv_special_values_and_padding(am):
    t, M = use(am, "perturbed8")
    m, n, k, lda, ldb, ldc = 3, 700, 90, 100, 710, 720
    A = normal(931, (m, lda))
    B = normal(932, (k, ldb))
    A[0, 5] = np.inf
    A[1, :] = 0.0
    A[1, 7] = np.nan
    A[2, 3] = np.float32(1.0e-41)       # subnormal: counts as zero
    B[5, 11] = 0.0                      # Inf x 0 -> NaN at (0, 11)
    B[9, 40] = -np.inf
    B[20, 300] = np.float32(3.0e38)     # with A[0, 20] the product overflows: the wave falls back
    A[0, 20] = np.float32(1.0e10)
    B[21, 600] = np.float32(1.0e-30)    # with A[2, 21] the product underflows to zero
    A[2, 21] = np.float32(1.0e-12)
    R, S = oracle.gemm(A[:, :k], B[:, :n], t, M)
    Cd = torch.full((m, ldc), 7.0, device="cuda")
    am.approx_gemm(0, 0, m, n, k, dev(A), lda, dev(B), ldb, Cd, ldc)
    Ch = host(Cd)
    with np.errstate(invalid="ignore"):
        gate(Ch[:, :n], R, S, what="gemv specials")
    assert np.all(Ch[:, n:] == 7.0)     # the padding of C is not written


def test_gemv_batched(am):
    t, M = use(am, "mitchell7")
    nb, n, k = 5, 300, 200
    As = [normal(940 + i, (1, k)) for i in range(nb)]
    Bs = [normal(950 + i, (k, n)) for i in range(nb)]
    Ad = dev(np.stack(As))
    Bd = dev(np.stack(Bs))
    C = torch.full((nb, 1, n), -1.0, device="cuda")
    am.approx_gemm_strided_batched(0, 0, 1, n, k, Ad, k, k, Bd, n, k * n, C, n, n, nb)
    got = host(C)
    for i in range(nb):
        R, S = oracle.gemm(As[i], Bs[i], t, M)
        gate(got[i], R, S, what=f"gemv strided batch {i}")
    C2 = torch.full((nb, 1, n), -1.0, device="cuda")
    ap = am.pointer_array([Ad[i].data_ptr() for i in range(nb)])
    bp = am.pointer_array([Bd[i].data_ptr() for i in range(nb)])
    cp = am.pointer_array([C2[i].data_ptr() for i in range(nb)])
    am.approx_gemm_batched(0, 0, 1, n, k, ap, k, bp, n, cp, n, nb)
    assert np.array_equal(host(C2), got)   # same kernel, same order


@pytest.mark.parametrize("m,transA", [(7, 0), (11, 1), (16, 0)])
def test_gemv_row_blocks_pointer_arrays(am, m, transA):
    """More than 4 rows through device pointer arrays: each entry's row blocks are
    offset from its own pointer; results equal the strided batch's bits."""
    t, M = use(am, "mitchell7")
    nb, n, k = 4, 500, 300
    ar, ac = (k, m) if transA else (m, k)
    As = np.stack([normal(1940 + i, (ar, ac)) for i in range(nb)])
    Bs = np.stack([normal(1950 + i, (k, n)) for i in range(nb)])
    Ad, Bd = dev(As), dev(Bs)
    C = torch.full((nb, m, n), -1.0, device="cuda")
    am.approx_gemm_strided_batched(transA, 0, m, n, k, Ad, ac, ar * ac, Bd, n, k * n, C, n, m * n, nb)
    got = host(C)
    for i in range(nb):
        R, S = oracle.gemm(As[i], Bs[i], t, M, transA=bool(transA))
        gate(got[i], R, S, what=f"row blocks batch {i}")
    order = [2, 0, 3, 1]
    C2 = torch.full((nb, m, n), -1.0, device="cuda")
    ap = am.pointer_array([Ad[i].data_ptr() for i in order])
    bp = am.pointer_array([Bd[i].data_ptr() for i in order])
    cp = am.pointer_array([C2[i].data_ptr() for i in order])
    am.approx_gemm_batched(transA, 0, m, n, k, ap, ac, bp, n, cp, n, nb)
    assert np.array_equal(host(C2), got)   # same kernel, same order


def test_gemv_8192_full_size(am):
    """Batch-1 inference through an 8192 x 8192 layer with the M = 8 perturbed
    table: the configuration `bench.py --gemv` times; every output checked."""
    t, M = use(am, "perturbed8")
    x = normal(961, (1, 8192))
    W = normal(962, (8192, 8192))
    R, S = oracle.gemm(x, W, t, M)
    gate(host(am.gemm(dev(x), dev(W))), R, S, what="gemv 8192")


def test_gemv_deterministic(am):
    use(am, "mitchell7")
    x = dev(normal(971, (2, 3000)))
    W = dev(normal(972, (3000, 2500)))
    c1 = host(am.gemm(x, W))
    c2 = host(am.gemm(x, W))
    assert np.array_equal(c1.view(np.uint32), c2.view(np.uint32))
