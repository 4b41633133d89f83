"""GPU parity: the HIP path (through the C ABI) against the oracle.

Products (GEMMs with k = 1) must be bit-exact; sums must pass the gate of
tests/parity.py (|c - r| <= 1e-5 * sum|products|). Inputs come from datagen;
expected values only from the oracle.
"""
import os

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one, special_values, splitmix64, uniform
from datagen import configs as cfg
from parity import gate, same_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def am():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import approximate_multiplier_dnn_amd as m
    return m


_TABLES = {}


def table(name):
    """(M, table) from the oracle's generator (the expected side)."""
    if name not in _TABLES:
        if name == "exact7":
            _TABLES[name] = (7, oracle.lut_generate(7, "exact"))
        elif name == "mitchell7":
            _TABLES[name] = (7, oracle.lut_generate(7, "mitchell"))
        elif name == "perturbed8":
            _TABLES[name] = (8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16)))
        elif name == "mitchell3":
            _TABLES[name] = (3, oracle.lut_generate(3, "mitchell"))
        elif name.startswith("arbitrary"):      # every entry a seeded random 16-bit word
            M = int(name[len("arbitrary"):])
            _TABLES[name] = (M, (splitmix64(7200 + M, 1 << (2 * M)) >> np.uint64(48)).astype(np.uint16))
        else:
            raise KeyError(name)
    return _TABLES[name]


def use(am, name):
    M, t = table(name)
    am.approx_lut_load(t, M)
    return M, t


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


class forced_checked:
    """Force the per-product checked path for the calls inside the block."""

    def __enter__(self):
        os.environ["APPROX_FORCE_CHECKED"] = "1"

    def __exit__(self, *a):
        os.environ.pop("APPROX_FORCE_CHECKED", None)


# ------------------------------------------------------------------ products

def _operand_values(M, exps):
    mant = np.arange(1 << M, dtype=np.uint32) << np.uint32(23 - M)
    # a set bit below the top M bits must be ignored by the table index
    low = np.uint32(1 << (22 - M)) if M < 23 else np.uint32(0)
    vals = [(s << 31) | (np.uint32(e) << 23) | mant | (low * ((mant >> np.uint32(23 - M)) & 1))
            for e in exps for s in (0, 1)]
    sp = special_values().view(np.uint32)
    return np.concatenate(vals + [sp]).astype(np.uint32)


ALL_WIDTHS = ["arbitrary1", "arbitrary2", "arbitrary4", "arbitrary5", "arbitrary6", "arbitrary8"]


@pytest.mark.parametrize("name", ["exact7", "mitchell7", "perturbed8", "mitchell3"] + ALL_WIDTHS)
@pytest.mark.parametrize("exps", ["moderate", "extreme", "moderate_checked"])
def test_products_bit_exact(am, name, exps):
    """C = a b^T with k = 1: every output is +0 + one approximate product."""
    M, t = use(am, name)
    e = [100, 127, 150] if exps.startswith("moderate") else [1, 2, 63, 64, 126, 127, 128, 190, 191, 253, 254]
    a = _operand_values(M, e)
    b = _operand_values(M, e[::-1])
    A = dev(a.view(np.float32).reshape(-1, 1))
    B = dev(b.view(np.float32).reshape(-1, 1))
    C = torch.empty((a.size, b.size), dtype=torch.float32, device="cuda")
    print(f"products {name} {exps}: {a.size} x {b.size}", flush=True)
    # B as a transposed k = 1 operand: the GEMM kernel for every row count
    # (the row-vector kernel has its own products tests)
    if exps == "moderate_checked":
        with forced_checked():
            am.approx_gemm(0, 1, a.size, b.size, 1, A, 1, B, 1, C, b.size)
    else:
        am.approx_gemm(0, 1, a.size, b.size, 1, A, 1, B, 1, C, b.size)
    got = host(C).view(np.uint32)
    want = oracle.amsim_bits(np.repeat(a, b.size), np.tile(b, a.size), t, M).reshape(a.size, b.size)
    want = np.where(want == 0x80000000, 0, want).astype(np.uint32)     # +0 + (-0) = +0
    gnan = np.isnan(got.view(np.float32))
    wnan = np.isnan(want.view(np.float32))
    assert np.array_equal(gnan, wnan)
    bad = np.count_nonzero(got[~gnan] != want[~wnan])
    assert bad == 0, f"{bad} products differ"


# ------------------------------------------------------------------ GEMM

GEMM_SHAPES = [
    (1, 1, 1), (7, 5, 3), (64, 64, 64), (65, 17, 129), (300, 33, 70), (513, 130, 257), (20, 300, 1000),
]


@pytest.mark.parametrize("transA,transB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_parity(am, shape, transA, transB):
    m, n, k = shape
    M, t = use(am, "mitchell7")
    seed = 7 * m + 13 * n + k + 100 * transA + 200 * transB
    A = normal(seed, (k, m) if transA else (m, k))
    B = normal(seed + 1, (n, k) if transB else (k, n))
    R, S = oracle.gemm(A, B, t, M, transA=bool(transA), transB=bool(transB))
    C = am.gemm(dev(A), dev(B), transA=bool(transA), transB=bool(transB))
    gate(host(C), R, S, what=f"gemm {shape} {transA}{transB}")


@pytest.mark.parametrize("name", ALL_WIDTHS)
def test_gemm_and_conv_every_table_width(am, name):
    """Tables of M = 1..8 with arbitrary entries (the LDS image's column
    stride and pad position follow M): a GEMM and a Conv2D forward pass."""
    M, t = use(am, name)
    A = normal(640 + M, (150, 333))
    B = normal(641 + M, (333, 90))
    R, S = oracle.gemm(A, B, t, M)
    gate(host(am.gemm(dev(A), dev(B))), R, S, what=f"gemm {name}")
    x = normal(642 + M, (2, 9, 11, 5))
    w = normal(643 + M, (3, 3, 5, 7))
    Y, YS = oracle.conv2d_fwd(x, w, t, M, (1, 2), (1, 1))
    gate(host(am.conv2d_fwd(dev(x), dev(w), (1, 2), (1, 1))), Y, YS, what=f"conv {name}")


def test_gemm_leading_dimensions_and_untouched_padding(am):
    M, t = use(am, "perturbed8")
    m, n, k, lda, ldb, ldc = 100, 37, 61, 70, 50, 45
    Ab = normal(1, (m, lda))
    Bb = normal(2, (k, ldb))
    R, S = oracle.gemm(Ab[:, :k], Bb[:, :n], t, M)
    Cd = torch.full((m, ldc), 7.0, device="cuda")
    am.approx_gemm(0, 0, m, n, k, dev(Ab), lda, dev(Bb), ldb, Cd, ldc)
    Ch = host(Cd)
    gate(Ch[:, :n], R, S, what="ld")
    assert np.all(Ch[:, n:] == 7.0)


@pytest.mark.parametrize("offset", [0, 1, 2])
@pytest.mark.parametrize("ld_extra", [0, 3, 4])
def test_gemm_source_alignment(am, offset, ld_extra):
    """Operands that start off a 16-byte boundary, or whose rows are not a
    multiple of 4 floats apart, against the same operands aligned: the decode
    reads them 4 at a time only where that is possible."""
    M, t = use(am, "mitchell7")
    m, n, k = 90, 75, 131
    lda, ldb = k + ld_extra, k + ld_extra
    seed = 500 + 10 * offset + ld_extra
    A = normal(seed, (m, k))
    Bt = normal(seed + 1, (n, k))
    bufA = np.zeros(offset + m * lda, np.float32)
    bufB = np.zeros(offset + n * ldb, np.float32)
    bufA[offset:].reshape(m, lda)[:, :k] = A
    bufB[offset:].reshape(n, ldb)[:, :k] = Bt
    dA, dB = dev(bufA), dev(bufB)
    C = torch.empty((m, n), dtype=torch.float32, device="cuda")
    am.approx_gemm(0, 1, m, n, k, dA[offset:], lda, dB[offset:], ldb, C, n)
    R, S = oracle.gemm(A, Bt, t, M, transB=True)
    gate(host(C), R, S, what=f"alignment {offset} {ld_extra}")
    ref = am.gemm(dev(A), dev(Bt), transB=True)
    assert np.array_equal(host(C).view(np.uint32), host(ref).view(np.uint32))


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8"])
def test_gemm_tail_tiles_split(am, name):
    """257-258 output tiles (one more than a round of resident workgroups):
    the full round's tiles are computed whole, only the last tile(s) in
    reduction chunks whose partials are summed afterwards. Checked on every
    output of the last 256 columns (where the split tiles lie) and on random
    outputs everywhere."""
    M, t = use(am, name)
    m, n, k = 512, 64 * 257, 1024
    A = normal(811, (m, k))
    B = normal(812, (k, n))
    C = host(am.gemm(dev(A), dev(B)))
    rr, cc = np.meshgrid(np.arange(m, dtype=np.int32), np.arange(n - 256, n, dtype=np.int32), indexing="ij")
    sr, sc = _sample_pairs(813, m, n, 4096)
    rows = np.concatenate([rr.ravel(), sr])
    cols = np.concatenate([cc.ravel(), sc])
    R, S = oracle.gemm_at(A, B, t, M, rows, cols)
    gate(C[rows, cols], R, S, what=f"tail split {name}")


@pytest.mark.parametrize("mode", ["pointers", "strided"])
def test_batched_tail_tiles_split(am, mode):
    """257 or 260 batch entries of one output tile each: the entries of the
    full round are computed whole, the last ones in reduction chunks (split
    partials summed per entry, outputs found through the pointer array or the
    batch stride)."""
    M, t = use(am, "mitchell7")
    m, n, k = 64, 16, 1024
    batch = 257 if mode == "pointers" else 260
    A = normal(821, (batch, m, k))
    B = normal(822, (batch, k, n))
    C = torch.full((batch, m, n + 2), -3.0, dtype=torch.float32, device="cuda")
    dA, dB = dev(A), dev(B)
    if mode == "pointers":
        order = [(7 * i) % batch for i in range(batch)]   # entries not in memory order
        pa = am.pointer_array([dA[i].data_ptr() for i in order])
        pb = am.pointer_array([dB[i].data_ptr() for i in order])
        pc = am.pointer_array([C[i].data_ptr() for i in order])
        am.approx_gemm_batched(0, 0, m, n, k, pa, k, pb, n, pc, n + 2, batch)
    else:
        am.approx_gemm_strided_batched(0, 0, m, n, k, dA, k, m * k, dB, n, k * n, C, n + 2, m * (n + 2), batch)
    got = host(C)
    for i in range(batch):
        R, S = oracle.gemm(A[i], B[i], t, M)
        gate(got[i][:, :n], R, S, what=f"{mode} entry {i}")
    assert np.all(got[:, :, n:] == -3.0)


def test_gemm_k_zero_and_empty(am):
    use(am, "mitchell7")
    C = torch.full((5, 6), 3.0, device="cuda")
    A = torch.ones((5, 1), device="cuda")
    B = torch.ones((1, 6), device="cuda")
    am.approx_gemm(0, 0, 5, 6, 0, A, 1, B, 6, C, 6)
    assert np.all(host(C) == 0)
    C.fill_(3.0)
    am.approx_gemm(0, 0, 0, 6, 4, A, 4, B, 6, C, 6)
    am.approx_gemm(0, 0, 5, 0, 4, A, 4, B, 6, C, 6)
    assert np.all(host(C) == 3.0)


def test_gemm_special_values_and_extremes(am):
    """Zeros, subnormals, Inf, NaN and exponents near the ends of the range
    (the checked path), against the oracle."""
    M, t = use(am, "exact7")
    m, n, k = 40, 24, 50
    A = normal(11, (m, k))
    B = normal(12, (k, n))
    A[3, :] = 0.0
    A[5, 7] = np.float32(1e-40)         # subnormal
    A[6, 2] = np.inf
    B[9, 4] = np.nan
    B[:, 10] = np.float32(1e35)         # large but the FP32 sums stay finite
    A[7, :] = np.float32(1e-30)
    B[:, 11] = np.float32(1e-20)        # products underflow
    A[8, 5] = np.float32(1e30)
    B[5, 12] = np.float32(1e30)         # one product overflows to +-Inf
    R, S = oracle.gemm(A, B, t, M)
    with np.errstate(invalid="ignore"):
        C = host(am.gemm(dev(A), dev(B)))
    gate(C, R, S, what="specials")


@pytest.mark.parametrize("name,shape", [
    ("perturbed8", (300, 150, 200)),      # GEMM kernel
    ("exact7", (64, 64, 64)),             # row-vector kernel (k * n <= 2^16: up to 64 rows)
    ("perturbed8", (48, 2048, 2048)),     # row-vector kernel (k * n >= 2^22), 12 row blocks
])
def test_fast_and_checked_paths_agree_bitwise(am, name, shape):
    use(am, name)
    m, n, k = shape
    A = dev(normal(21 + m, (m, k)))
    B = dev(normal(22 + n, (k, n)))
    C1 = host(am.gemm(A, B))
    with forced_checked():
        C2 = host(am.gemm(A, B))
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))


def test_deterministic_including_split_reduction(am):
    use(am, "mitchell7")
    for (m, n, k) in ((64, 48, 60000), (1024, 1024, 512)):
        A = dev(normal(31, (m, k)))
        B = dev(normal(32, (k, n)))
        C1 = host(am.gemm(A, B))
        C2 = host(am.gemm(A, B))
        assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
    # split reductions still meet the gate: 16 rows run in the row-vector
    # kernel (its chunk partials summed by the reduction kernel), 100 rows in
    # the GEMM kernel (one row tile, its reduction split over the chunks)
    M, t = table("mitchell7")
    for m, what in ((16, "split, row-vector kernel"), (100, "split, GEMM kernel")):
        A = normal(33, (m, 40000))
        B = normal(34, (40000, 20))
        R, S = oracle.gemm(A, B, t, M)
        gate(host(am.gemm(dev(A), dev(B))), R, S, what=what)


def test_strided_batched_heads(am):
    """Attention-style batched products over heads inside a fused QKV buffer."""
    M, t = use(am, "mitchell7")
    T, H, dh = 70, 3, 16
    qkv = normal(41, (T, 3 * H * dh))
    S_out = torch.empty((H, T, T), dtype=torch.float32, device="cuda")
    q = dev(qkv)
    # S_h = Q_h K_h^T: A = Q_h (ld 3*H*dh), B = K_h stored row-major, transB
    am.approx_gemm_strided_batched(0, 1, T, T, dh, q, 3 * H * dh, dh, q[:, H * dh:], 3 * H * dh, dh,
                                   S_out, T, T * T, H)
    got = host(S_out)
    for h in range(H):
        Qh = qkv[:, h * dh:(h + 1) * dh]
        Kh = qkv[:, H * dh + h * dh: H * dh + (h + 1) * dh]
        R, S = oracle.gemm(Qh, Kh, t, M, transB=True)
        gate(got[h], R, S, what=f"head {h}")


def test_batched_by_pointer_arrays(am):
    """Matrices at unrelated places in different buffers, one call."""
    M, t = use(am, "mitchell7")
    m, n, k = 37, 29, 45
    bufA = normal(61, (5000,))
    bufB = normal(62, (7000,))
    offsA = [0, 1700, 3011]
    offsB = [4000, 13, 2500]
    As = [bufA[o:o + m * k].reshape(m, k) for o in offsA]
    Bs = [bufB[o:o + k * n].reshape(k, n) for o in offsB]
    dA, dB = dev(bufA), dev(bufB)
    C = torch.full((3, m, n + 3), -1.0, device="cuda")
    pa = am.pointer_array([dA.data_ptr() + 4 * o for o in offsA])
    pb = am.pointer_array([dB.data_ptr() + 4 * o for o in offsB])
    pc = am.pointer_array([C[i].data_ptr() for i in range(3)])
    am.approx_gemm_batched(0, 0, m, n, k, pa, k, pb, n, pc, n + 3, 3)
    got = host(C)
    for i in range(3):
        R, S = oracle.gemm(As[i], Bs[i], t, M)
        gate(got[i][:, :n], R, S, what=f"ptr batch {i}")
        assert np.all(got[i][:, n:] == -1.0)


# ------------------------------------------------------------------ Conv2D

CONV_GEOMS = [
    # N, H, W, C, K, R, S, stride, pad
    (2, 8, 8, 4, 5, 3, 3, (1, 1), (1, 1)),
    (1, 9, 7, 3, 2, 3, 3, (2, 2), (1, 1)),
    (2, 6, 10, 5, 3, 3, 2, (2, 1), (0, 1)),
    (1, 7, 7, 2, 4, 1, 1, (1, 1), (0, 0)),
    (1, 5, 6, 3, 3, 3, 3, (1, 2), (2, 1)),
    (1, 10, 9, 2, 2, 4, 3, (3, 2), (1, 0)),
    (3, 12, 12, 16, 24, 3, 3, (1, 1), (1, 1)),
    (2, 9, 11, 7, 33, 5, 5, (1, 1), (2, 2)),
    (2, 16, 16, 64, 64, 3, 3, (1, 1), (1, 1)),
    (2, 5, 6, 3, 4, 1, 2, (2, 2), (2, 3)),     # padding wider than the filter: all-zero border outputs
    (1, 1, 1, 3, 2, 3, 3, (1, 1), (1, 1)),     # a 1 x 1 image under a 3 x 3 filter
    (1, 4, 5, 6, 3, 4, 5, (4, 5), (0, 0)),     # one output pixel, stride equal to the filter
]


@pytest.mark.parametrize("geom", CONV_GEOMS)
def test_conv_parity(am, geom):
    N, H, W, C, K, R, S, stride, pad = geom
    M, t = use(am, "mitchell7")
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(51, (N, H, W, C))
    w = normal(52, (R, S, C, K))
    dy = normal(53, (N, P, Q, K))
    print(f"conv {geom}", flush=True)
    Y, YS = oracle.conv2d_fwd(x, w, t, M, stride, pad)
    gate(host(am.conv2d_fwd(dev(x), dev(w), stride, pad)), Y, YS, what="fwd")
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, t, M, stride, pad)
    gate(host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, stride, pad)), DX, DXS, what="dgrad")
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, t, M, stride, pad)
    gate(host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, stride, pad)), DW, DWS, what="wgrad")


def test_conv_padding_multiplies_zero(am):
    """An infinite weight facing padding gives NaN, as IM2COL + GEMM would."""
    M, t = use(am, "exact7")
    x = np.ones((1, 4, 4, 1), np.float32)
    w = np.ones((3, 3, 1, 1), np.float32)
    w[0, 0, 0, 0] = np.inf
    Y, YS = oracle.conv2d_fwd(x, w, t, M, (1, 1), (1, 1))
    with np.errstate(invalid="ignore"):
        gate(host(am.conv2d_fwd(dev(x), dev(w), (1, 1), (1, 1))), Y, YS, what="pad-inf")


# ------------------------------------------------------------------ the five workloads

def _sample_pairs(seed, m, n, count):
    r = splitmix64(seed, 2 * count)
    rows = (r[0::2] % np.uint64(m)).astype(np.int32)
    cols = (r[1::2] % np.uint64(n)).astype(np.int32)
    return rows, cols


def test_workload1_gemm64(am):
    M, t = use(am, "exact7")
    A, B = cfg.gemm_square(1, 64)
    R, S = oracle.gemm(A, B, t, M)
    gate(host(am.gemm(dev(A), dev(B))), R, S, what="w1")


def test_workload2_mlp_all_gemms(am):
    M, t = use(am, "mitchell7")
    layers = cfg.mlp_tensors()
    for (name, ta, tb, m, n, k, an, bn) in cfg.mlp_gemms():
        X, W, dY = layers[int(name[-1])]
        ops = {"X": X, "W": W, "dY": dY}
        A, B = ops[an], ops[bn]
        print(f"mlp {name} {m}x{n}x{k}", flush=True)
        R, S = oracle.gemm(A, B, t, M, transA=bool(ta), transB=bool(tb))
        C = host(am.gemm(dev(A), dev(B), transA=bool(ta), transB=bool(tb)))
        assert C.shape == (m, n)
        gate(C, R, S, what=f"mlp {name}")


def _rows_cols_sample(seed, m, n, n_rows=64, n_cols=64, n_rand=4096):
    """The full-size sample: n_rows full rows and n_cols full columns (the
    first and last of each included) and n_rand random outputs, as flat
    (row, column) arrays."""
    r = splitmix64(seed, n_rows + n_cols)
    rsel = np.unique(np.concatenate([[0, m - 1], (r[:n_rows - 2] % np.uint64(m)).astype(np.int64)]))
    csel = np.unique(np.concatenate([[0, n - 1], (r[n_rows:n_rows + n_cols - 2] % np.uint64(n)).astype(np.int64)]))
    rows = [np.repeat(rsel, n), np.repeat(np.arange(m), csel.size)]
    cols = [np.tile(np.arange(n), rsel.size), np.tile(csel, m)]
    rr, cc = _sample_pairs(seed + 1, m, n, n_rand)
    rows = np.concatenate(rows + [rr]).astype(np.int32)
    cols = np.concatenate(cols + [cc]).astype(np.int32)
    return rows, cols, rsel.size, csel.size


def _check_gemm_sample(am, C, A, B, t, M, rows, cols, what, transA=False, transB=False, batch=1, b=0):
    """Sampled outputs of a GEMM: the double-precision gate and the FP32
    sums in the reported order, bit for bit (threaded oracle driver)."""
    m, n = C.shape
    k = A.shape[0] if transA else A.shape[1]
    th = oracle.default_threads()
    R, S = oracle.gemm_at(A, B, t, M, rows, cols, transA=transA, transB=transB, threads=th)
    gate(C[rows, cols], R, S, what=what)
    L = am.approx_gemm_chunks(int(transA), int(transB), m, n, k, batch, b, rows, cols)
    F = oracle.gemm_f32_at(A, B, t, M, rows, cols, np.maximum(L, 1), transA=transA, transB=transB, threads=th)
    same_bits(C[rows, cols], F, what=what)


def test_workload3_conv_full_size(am):
    """The 3 x 3 Conv2D workload (NHWC 128 x 32 x 32 x 64 -> 64, Mitchell
    M = 7) in the launch configuration bench.py times: every output of all
    three passes equals the FP32 sums in the reported order bit for bit; every
    weight-gradient output and 4,096 random outputs of the other passes pass
    the double-precision gate."""
    import time
    M, t = use(am, "mitchell7")
    sh = cfg.CONV_SHAPE
    x, w, dy = cfg.conv_tensors()
    st, pd = sh["stride"], sh["pad"]
    geom = (sh["N"], sh["H"], sh["W"], sh["C"], sh["K"], sh["R"], sh["S"], st, pd)
    y = host(am.conv2d_fwd(dev(x), dev(w), st, pd)).ravel()
    dx = host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, st, pd)).ravel()
    dw = host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, st, pd)).ravel()
    th = oracle.default_threads()
    r = splitmix64(3301, 4096)
    for name, full, fn, args, t1, t2 in (
        ("fwd", y, oracle.conv2d_fwd, (x, w), x, w),
        ("dgrad", dx, oracle.conv2d_dgrad, (dy, w, x.shape), dy, w),
        ("wgrad", dw, oracle.conv2d_wgrad, (x, dy, w.shape), x, dy),
    ):
        t0 = time.time()
        if name == "wgrad":
            idx = np.arange(full.size, dtype=np.int64)
        else:
            idx = (r % np.uint64(full.size)).astype(np.int64)
            edges = np.array([0, full.size - 1, 31 * 64, 32 * 64 * 31, 32 * 32 * 64 - 1]) % full.size
            idx = np.concatenate([idx, edges])   # corners and image borders
        R, S = fn(*args, t, M, st, pd, idx=idx, threads=th)
        gate(full[idx], R, S, what=f"w3 {name}")
        every = np.arange(full.size, dtype=np.int64)
        L = am.approx_conv2d_chunks(name, *geom[:7], st, pd, every)
        F = oracle.conv2d_f32(name, t1, t2, geom, t, M, L, threads=th)
        same_bits(full, F, what=f"w3 {name}")
        print(f"w3 {name}: {idx.size} outputs gated, {full.size} bit-exact, {time.time() - t0:.1f} s", flush=True)


def test_conv_tail_tiles_split(am):
    """A 3 x 3 forward and input-gradient pass over 130 images of 32 x 32:
    133,120 output pixels make 260 row tiles, so the last 4 tiles (the last
    two images) are split and their partials summed. Every output of those
    images is checked, and random outputs elsewhere."""
    M, t = use(am, "mitchell7")
    N, H, W, C, K = 130, 32, 32, 64, 64
    x = normal(831, (N, H, W, C))
    w = normal(832, (3, 3, C, K), std=0.06)
    dy = normal(833, (N, H, W, K))
    y = host(am.conv2d_fwd(dev(x), dev(w), (1, 1), (1, 1))).ravel()
    dx = host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, (1, 1), (1, 1))).ravel()
    per_image = H * W * K
    tail = np.arange((N - 2) * per_image, N * per_image, dtype=np.int64)
    r = splitmix64(834, 2048)
    for name, full, fn, args in (("fwd", y, oracle.conv2d_fwd, (x, w)),
                                 ("dgrad", dx, oracle.conv2d_dgrad, (dy, w, x.shape))):
        idx = np.concatenate([tail, (r % np.uint64(full.size)).astype(np.int64)])
        R, S = fn(*args, t, M, (1, 1), (1, 1), idx=idx)
        gate(full[idx], R, S, what=f"conv tail {name}")


def test_workload4_gemm8192_sampled(am):
    """The headline GEMM (8192^3, M = 8 perturbed table) in the launch
    configuration bench.py times: 64 full rows, 64 full columns and 4,096
    random outputs (the first and last row and column included) against the
    double-precision gate and, bit for bit, the FP32 sums in the reported
    order."""
    import time
    M, t = use(am, "perturbed8")
    A, B = cfg.gemm_square(4, 8192)
    print("w4: gemm 8192^3", flush=True)
    C = host(am.gemm(dev(A), dev(B)))
    rows, cols, nr, nc = _rows_cols_sample(4401, 8192, 8192)
    t0 = time.time()
    Bt = np.ascontiguousarray(B.T)            # the same op(B), read along its columns
    _check_gemm_sample(am, C, A, Bt, t, M, rows, cols, "w4", transB=True)
    print(f"w4: {nr} rows, {nc} columns, {rows.size} outputs checked in {time.time() - t0:.1f} s", flush=True)


def test_gemm8192_exact_table_every_output(am):
    """8192^3 with the exact M = 7 table: every approximate product is then
    the exact product of the operands truncated to 7 fraction bits (no
    N(0, 1) product leaves the range), so every one of the 67 M outputs must
    lie within the gate of the float64 product of the truncated matrices
    (a library routine: torch's float64 matmul)."""
    M, t = use(am, "exact7")
    A, B = cfg.gemm_square(4, 8192)
    mask = np.uint32(0xFFFFFFFF ^ ((1 << (23 - M)) - 1))
    At = (A.view(np.uint32) & mask).view(np.float32)
    Bt = (B.view(np.uint32) & mask).view(np.float32)
    print("gemm 8192^3, exact M = 7 table", flush=True)
    dA, dB = dev(A), dev(B)
    C = am.gemm(dA, dB)
    del dA, dB
    dAt, dBt = dev(At).double(), dev(Bt).double()
    R = torch.matmul(dAt, dBt)
    S = torch.matmul(dAt.abs(), dBt.abs())
    del dAt, dBt
    err = ((C.double() - R).abs() / S).max().item()
    assert err <= 1e-5, err


def test_conv_exact_table_every_output(am):
    """The 3 x 3 Conv2D workload (NHWC 128 x 32 x 32 x 64 -> 64) with the
    exact M = 7 table: every output of the forward, input-gradient and
    weight-gradient passes against the float64 convolution of the truncated
    tensors (IM2COL and matrix products in float64, padding slots zero), the
    same property as for the 8192^3 GEMM above."""
    import torch.nn.functional as F
    M, t = use(am, "exact7")
    sh = cfg.CONV_SHAPE
    x, w, dy = cfg.conv_tensors()
    st, pd = sh["stride"], sh["pad"]
    N, H, W, C, K, R, S_ = sh["N"], sh["H"], sh["W"], sh["C"], sh["K"], sh["R"], sh["S"]
    print("conv 3x3 workload, exact M = 7 table", flush=True)
    y = am.conv2d_fwd(dev(x), dev(w), st, pd)
    dx = am.conv2d_dgrad(dev(dy), dev(w), x.shape, st, pd)
    dw = am.conv2d_wgrad(dev(x), dev(dy), w.shape, st, pd)
    mask = np.uint32(0xFFFFFFFF ^ ((1 << (23 - M)) - 1))
    trunc = lambda a: dev((a.view(np.uint32) & mask).view(np.float32)).double()
    xt, wt, dyt = trunc(x), trunc(w), trunc(dy)
    L = H * W                                   # stride 1, pad 1: P x Q = H x W
    Wm = wt.permute(2, 0, 1, 3).reshape(C * R * S_, K)           # rows (c, r, s)
    dym = dyt.reshape(N, L, K)

    def check(got, ref, mag, what):
        err = ((got.double() - ref).abs() / mag).max().item()
        assert err <= 1e-5, (what, err)

    for sign in (1, -1):      # sign 1: values; -1: magnitudes (the gate's sum of |products|)
        f = (lambda v: v) if sign == 1 else torch.abs
        cols = F.unfold(f(xt).permute(0, 3, 1, 2), (R, S_), padding=pd, stride=st)   # N x (C R S) x L
        Y = (cols.transpose(1, 2) @ f(Wm)).reshape(N, H, W, K)
        DW = (cols.permute(1, 0, 2).reshape(C * R * S_, N * L) @ f(dym).reshape(N * L, K))
        DW = DW.reshape(C, R, S_, K).permute(1, 2, 0, 3)
        DX = F.fold((f(dym) @ f(Wm).T).transpose(1, 2), (H, W), (R, S_), padding=pd, stride=st).permute(0, 2, 3, 1)
        del cols
        if sign == 1:
            refs = (Y, DX, DW)
        else:
            check(y, refs[0], Y, "fwd")
            check(dx, refs[1], DX, "dgrad")
            check(dw, refs[2], DW, "wgrad")


def test_workload5_attention_stages(am):
    """The four approximate GEMM stages of multi-head attention at the
    workload's shapes, each called as bench.py calls it (softmax
    probabilities are synthetic: row-normalised exponentials of normal
    draws). Projections: 64 full rows, 64 full columns and 4,096 random
    outputs; QK^T and P V: every output of 16 (sequence, head) pairs, the
    first and the last included; all against the double-precision gate and,
    bit for bit, the FP32 sums in the reported order."""
    M, t = use(am, "mitchell7")
    sh = cfg.MHA_SHAPE
    Bz, T, D, H = sh["batch"], sh["seq"], sh["d_model"], sh["heads"]
    dh = D // H
    X, Wqkv, Wo = cfg.mha_tensors()
    # stage 1: QKV projection
    qkv = host(am.gemm(dev(X), dev(Wqkv)))
    rows, cols, _, _ = _rows_cols_sample(5501, Bz * T, 3 * D)
    _check_gemm_sample(am, qkv, X, Wqkv, t, M, rows, cols, "w5 qkv")
    # stage 2: scores for every (sequence, head) pair in one pointer-array
    # call, on a synthetic fused QKV buffer
    qk = normal(5502, (Bz * T, 3 * D), std=0.5)
    q = dev(qk)
    S_d = torch.empty((Bz, H, T, T), dtype=torch.float32, device="cuda")
    pairs = [(b, h) for b in range(Bz) for h in range(H)]
    f = 4
    qp = am.pointer_array([q.data_ptr() + f * (b * T * 3 * D + h * dh) for b, h in pairs])
    kp = am.pointer_array([q.data_ptr() + f * (b * T * 3 * D + D + h * dh) for b, h in pairs])
    sp = am.pointer_array([S_d.data_ptr() + f * (b * H + h) * T * T for b, h in pairs])
    am.approx_gemm_batched(0, 1, T, T, dh, qp, 3 * D, kp, 3 * D, sp, T, len(pairs))
    Sc = host(S_d)
    pick = [0, len(pairs) - 1] + [int(v) for v in splitmix64(5503, 14) % np.uint64(len(pairs) - 2) + np.uint64(1)]
    full_r, full_c = np.meshgrid(np.arange(T, dtype=np.int32), np.arange(T, dtype=np.int32), indexing="ij")
    for e in pick:
        b, h = pairs[e]
        rows_ = qk[b * T:(b + 1) * T]
        Qh, Kh = rows_[:, h * dh:(h + 1) * dh], rows_[:, D + h * dh: D + (h + 1) * dh]
        _check_gemm_sample(am, Sc[b, h], Qh, Kh, t, M, full_r.ravel(), full_c.ravel(), f"w5 qk b{b} h{h}",
                           transB=True, batch=len(pairs), b=e)
    # stage 3: P V for every (sequence, head) pair in one pointer-array call
    z = normal(5510, (len(pairs), T, T))
    P = np.exp(z - z.max(axis=2, keepdims=True))
    P = (P / P.sum(axis=2, keepdims=True)).astype(np.float32)
    del z
    V = normal(5511, (Bz * T, 3 * D))         # the V columns of a fused QKV buffer
    dP, dV = dev(P), dev(V)
    O_d = torch.empty((Bz * T, D), dtype=torch.float32, device="cuda")
    pp = am.pointer_array([dP.data_ptr() + f * e * T * T for e in range(len(pairs))])
    vp = am.pointer_array([dV.data_ptr() + f * (b * T * 3 * D + 2 * D + h * dh) for b, h in pairs])
    op = am.pointer_array([O_d.data_ptr() + f * (b * T * D + h * dh) for b, h in pairs])
    am.approx_gemm_batched(0, 0, T, dh, T, pp, T, vp, 3 * D, op, D, len(pairs))
    O = host(O_d)
    full_r, full_c = np.meshgrid(np.arange(T, dtype=np.int32), np.arange(dh, dtype=np.int32), indexing="ij")
    for e in pick:
        b, h = pairs[e]
        Vh = V[b * T:(b + 1) * T, 2 * D + h * dh: 2 * D + (h + 1) * dh]
        Oh = O[b * T:(b + 1) * T, h * dh:(h + 1) * dh]
        _check_gemm_sample(am, Oh, P[e], Vh, t, M, full_r.ravel(), full_c.ravel(), f"w5 pv b{b} h{h}",
                           batch=len(pairs), b=e)
    del P, dP
    # stage 4: output projection
    Oin = normal(5530, (Bz * T, D), std=0.3)
    Y = host(am.gemm(dev(Oin), dev(Wo)))
    rows, cols, _, _ = _rows_cols_sample(5531, Bz * T, D)
    _check_gemm_sample(am, Y, Oin, Wo, t, M, rows, cols, "w5 out")


# ------------------------------------------------------------------ API

def test_no_table_after_release(am):
    am.approx_release()
    A = torch.ones((4, 4), device="cuda")
    with pytest.raises(am.ApproxError) as e:
        am.gemm(A, A)
    assert e.value.status == am.APPROX_ENOLUT
    use(am, "mitchell7")
    assert am.approx_lut_bits() == 7
