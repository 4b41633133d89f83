"""GPU parity on seeded random cases: GEMM shapes, transposes, leading
dimensions, batches, tables (M = 3, 7, 8, 10 and the native multiplier),
exponent widths of the multiplier's format (8, 6, 5), operand scales that
push products out of the format's range, and special values; then Conv2D
geometries (strides, paddings, filter sizes, channel counts) through all
three passes. Every case is drawn from its own seed, so a failure names a
case that can be rerun alone.

Expected values come from the oracle only (ApproxTrain, arXiv 2209.04161,
Algorithm 2 for each product; GEMM and Conv2D as sums of those products).
Sums must pass the gate of tests/parity.py against the double-precision sums,
and equal bit for bit the oracle's FP32 sums in the order the library
reports (approx_gemm_chunks / approx_conv2d_chunks); outputs outside
op(A) op(B)'s extent (the padding of C) must be left untouched.
"""
import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one, special_values, splitmix64
from parity import gate, same_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TABLE_NAMES = ["mitchell7", "perturbed8", "mitchell3", "arbitrary10", "native"]
_TABLES = {}


def table(name):
    if name not in _TABLES:
        if name == "mitchell7":
            _TABLES[name] = (7, oracle.lut_generate(7, "mitchell"))
        elif name == "perturbed8":
            _TABLES[name] = (8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16)))
        elif name == "mitchell3":
            _TABLES[name] = (3, oracle.lut_generate(3, "mitchell"))
        elif name == "arbitrary10":       # every entry a seeded random 16-bit word
            _TABLES[name] = (10, (splitmix64(7010, 1 << 20) >> np.uint64(48)).astype(np.uint16))
        else:
            _TABLES[name] = (0, None)
    return _TABLES[name]


@pytest.fixture(scope="module")
def am():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import approximate_multiplier_dnn_amd as m
    yield m
    m.approx_exponent_bits_set(8)
    m.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)


def use(am, name, E):
    M, t = table(name)
    if name == "native":
        am.approx_native_load()
    else:
        am.approx_lut_load(t, M)
    am.approx_exponent_bits_set(E)
    return M, t


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# Zeros, subnormals, infinities and NaNs (special_values() less its large
# finite values: sums of products near the FP32 maximum overflow the FP32
# accumulator on the way, which a float64 sum of the same products does not
# show; k = 1 tests cover those products one by one).
SPECIALS = special_values()[[0, 1, 2, 3, 4, 19, 20, 21, 22, 23]]


def operand(seed, shape, scale_exp, special):
    """N(0, 1) values times 2^scale_exp; with `special`, about 1 in 300
    entries replaced by a special value (+-0, subnormal, +-Inf, NaN)."""
    x = normal(seed, shape) * np.float32(2.0 ** scale_exp)
    if special:
        flat = x.reshape(-1)
        r = splitmix64(seed + 77, flat.size)
        hit = (r % np.uint64(300)) == np.uint64(0)
        flat[hit] = SPECIALS[(r[hit] >> np.uint64(20)) % np.uint64(SPECIALS.size)]
    return x


# ---------------------------------------------------------------- GEMM

def gemm_case(i):
    g = np.random.default_rng(91000 + i)
    name = TABLE_NAMES[i % len(TABLE_NAMES)]
    E = 8 if name == "native" else int(g.choice([8, 8, 6, 5]))
    m = int(g.choice([1, 2, 3, 4, g.integers(5, 300), g.integers(300, 1300)]))
    n = int(g.choice([g.integers(1, 300), g.integers(300, 800)]))
    k = int(g.choice([1, 2, g.integers(3, 64), g.integers(64, 700), g.integers(700, 3000)]))
    while m * n * k > 60_000_000:            # the oracle's share stays within seconds
        k = max(1, k // 2)
    tA, tB = int(g.integers(2)), int(g.integers(2))
    batch = int(g.choice([1, 1, 2, 3]))
    pads = [int(g.choice([0, 0, 1, 3, 8])) for _ in range(3)]
    # scales: mostly moderate; some push products past the format's bounds
    sa, sb = [int(g.choice([0, 0, 0, -20, 20, -60, 50])) for _ in range(2)]
    if E < 8:
        sa, sb = sa // 8, sb // 8
    special = bool(g.integers(4) == 0)
    return dict(i=i, name=name, E=E, m=m, n=n, k=k, tA=tA, tB=tB, batch=batch, pads=pads, sa=sa, sb=sb,
                special=special)


GEMM_CASES = [gemm_case(i) for i in range(120)]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: f"g{c['i']}-{c['name']}-E{c['E']}")
def test_random_gemm(am, case):
    c = case
    print(f"random gemm case {c}", flush=True)
    M, t = use(am, c["name"], c["E"])
    m, n, k, batch = c["m"], c["n"], c["k"], c["batch"]
    ar, ac = (k, m) if c["tA"] else (m, k)
    br, bc = (n, k) if c["tB"] else (k, n)
    lda, ldb, ldc = ac + c["pads"][0], bc + c["pads"][1], n + c["pads"][2]
    sA, sB, sC = ar * lda + 5, br * ldb + 3, m * ldc + 7      # batch strides, off the rows' alignment
    seed = 300000 + 10 * c["i"]
    Abuf = operand(seed, (batch * sA,), c["sa"], c["special"])
    Bbuf = operand(seed + 1, (batch * sB,), c["sb"], c["special"])
    Cd = torch.full((batch * sC,), 7.0, dtype=torch.float32, device="cuda")
    dA, dB = dev(Abuf), dev(Bbuf)
    if batch == 1:
        am.approx_gemm(c["tA"], c["tB"], m, n, k, dA, lda, dB, ldb, Cd, ldc)
    else:
        am.approx_gemm_strided_batched(c["tA"], c["tB"], m, n, k, dA, lda, sA, dB, ldb, sB, Cd, ldc, sC, batch)
    got = host(Cd)
    for b in range(batch):
        A = Abuf[b * sA: b * sA + ar * lda].reshape(ar, lda)[:, :ac]
        B = Bbuf[b * sB: b * sB + br * ldb].reshape(br, ldb)[:, :bc]
        R, S = oracle.gemm(A, B, t, M, transA=bool(c["tA"]), transB=bool(c["tB"]), E=c["E"])
        Cb = got[b * sC: b * sC + m * ldc].reshape(m, ldc)
        with np.errstate(invalid="ignore", over="ignore"):
            gate(Cb[:, :n], R, S, what=f"random gemm {c['i']} batch {b}")
        # bit for bit against the FP32 sums in the library's reported order
        rows, cols = np.meshgrid(np.arange(m, dtype=np.int32), np.arange(n, dtype=np.int32), indexing="ij")
        rows, cols = rows.ravel(), cols.ravel()
        L = am.approx_gemm_chunks(c["tA"], c["tB"], m, n, k, batch, b, rows, cols)
        F = oracle.gemm_f32_at(A, B, t, M, rows, cols, np.maximum(L, 1), transA=bool(c["tA"]),
                               transB=bool(c["tB"]), E=c["E"])
        same_bits(Cb[:, :n], F, what=f"random gemm {c['i']} batch {b}", zero_sign=t is not None)
        assert np.all(Cb[:, n:] == 7.0)
        gap = got[b * sC + m * ldc: (b + 1) * sC] if b + 1 < batch else got[b * sC + m * ldc:]
        assert np.all(gap == 7.0)


# ---------------------------------------------------------------- Conv2D

def conv_case(i):
    g = np.random.default_rng(92000 + i)
    name = TABLE_NAMES[i % len(TABLE_NAMES)]
    E = 8 if name == "native" else int(g.choice([8, 8, 5]))
    while True:
        N = int(g.integers(1, 4))
        H, W = int(g.choice([g.integers(1, 18), g.integers(18, 40)])), int(g.choice([g.integers(1, 18), g.integers(18, 40)]))
        C, K = int(g.choice([1, 3, g.integers(1, 40), g.integers(40, 80)])), int(g.choice([1, 4, g.integers(1, 40), g.integers(40, 80)]))
        R, S = int(g.integers(1, 6)), int(g.integers(1, 6))
        sh, sw = int(g.integers(1, 4)), int(g.integers(1, 4))
        ph, pw = int(g.integers(0, R)), int(g.integers(0, S))
        if H + 2 * ph >= R and W + 2 * pw >= S:
            break
    special = bool(g.integers(4) == 0)
    return dict(i=i, name=name, E=E, N=N, H=H, W=W, C=C, K=K, R=R, S=S, stride=(sh, sw), pad=(ph, pw),
                special=special)


CONV_CASES = [conv_case(i) for i in range(50)]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: f"c{c['i']}-{c['name']}-E{c['E']}")
def test_random_conv(am, case):
    c = case
    print(f"random conv case {c}", flush=True)
    M, t = use(am, c["name"], c["E"])
    N, H, W, C, K, R, S = c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"]
    st, pd, E = c["stride"], c["pad"], c["E"]
    P, Q = oracle.conv_out_hw(H, W, R, S, st, pd)
    seed = 400000 + 10 * c["i"]
    x = operand(seed, (N, H, W, C), 0, c["special"])
    w = operand(seed + 1, (R, S, C, K), -2, c["special"])
    dy = operand(seed + 2, (N, P, Q, K), 0, c["special"])
    geom = (N, H, W, C, K, R, S, st, pd)
    with np.errstate(invalid="ignore", over="ignore"):
        Y, YS = oracle.conv2d_fwd(x, w, t, M, st, pd, E=E)
        y = host(am.conv2d_fwd(dev(x), dev(w), st, pd))
        gate(y, Y, YS, what=f"random conv {c['i']} fwd")
        DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, t, M, st, pd, E=E)
        dx = host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, st, pd))
        gate(dx, DX, DXS, what=f"random conv {c['i']} dgrad")
        DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, t, M, st, pd, E=E)
        dw = host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, st, pd))
        gate(dw, DW, DWS, what=f"random conv {c['i']} wgrad")
    # bit for bit against the FP32 sums in the library's reported order
    for pname, got, t1, t2 in (("fwd", y, x, w), ("dgrad", dx, dy, w), ("wgrad", dw, x, dy)):
        idx = np.arange(got.size, dtype=np.int64)
        L = am.approx_conv2d_chunks(pname, N, H, W, C, K, R, S, st, pd, idx)
        F = oracle.conv2d_f32(pname, t1, t2, geom, t, M, L, idx=idx, E=E)
        same_bits(got, F, what=f"random conv {c['i']} {pname}", zero_sign=t is not None)
