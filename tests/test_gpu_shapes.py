"""Every workgroup shape of the GEMM kernel on dense GEMMs, forced through
APPROX_KERNEL_SHAPE: shape 0 (8 waves x 4 rows per lane, 256 x 128 tiles at
most), shape 1 (12 waves x 3 rows) and shape 2 (8 waves x 2 rows, the tiles
that small dense GEMMs take by default). Each forced call must give the
oracle's FP32 sums in the summation order the library reports for that
shape (approx_gemm_chunks under the same setting), bit for bit, on whole
rows and columns and a random sample: tables in LDS (M = 7, M = 8 with its
second copies) and in global memory (M = 10), all four transposes, split
and whole tiles, ragged edges; and the convolution's three passes, whose
forward and input-gradient passes run in vector mode like the GEMMs.
"""
import os

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one, splitmix64
from parity import same_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TABLES = {
    "mitchell7": lambda: (7, oracle.lut_generate(7, "mitchell")),
    "perturbed8": lambda: (8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16))),
    "arbitrary10": lambda: (10, (splitmix64(7010, 1 << 20) >> np.uint64(48)).astype(np.uint16)),
}

CASES = [
    # (transA, transB, m, n, k)
    (0, 0, 256, 1024, 784),
    (0, 1, 300, 200, 517),
    (1, 0, 784, 130, 256),
    (1, 1, 97, 333, 1200),
    (0, 0, 1000, 64, 40),
]


@pytest.fixture(scope="module")
def am():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import approximate_multiplier_dnn_amd as m
    yield m
    os.environ.pop("APPROX_KERNEL_SHAPE", None)
    m.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("shape", ["0", "1", "2"])
@pytest.mark.parametrize("name", sorted(TABLES))
@pytest.mark.parametrize("case", range(len(CASES)))
def test_forced_shape_gives_the_fp32_order_sums(am, shape, name, case):
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    tA, tB, m, n, k = CASES[case]
    A = normal(9400 + case, (k, m) if tA else (m, k))
    B = normal(9410 + case, (n, k) if tB else (k, n))
    C = torch.full((m, n), -2.0, dtype=torch.float32, device="cuda")
    print(f"shape {shape} {name} {CASES[case]}", flush=True)
    os.environ["APPROX_KERNEL_SHAPE"] = shape
    try:
        am.approx_gemm(tA, tB, m, n, k, dev(A), A.shape[1], dev(B), B.shape[1], C, n)
        torch.cuda.synchronize()
        r = np.arange(m, dtype=np.int32)
        c = np.arange(n, dtype=np.int32)
        rows = np.concatenate([np.full(n, m - 1, np.int32), r, (splitmix64(9420 + case, 600) % np.uint64(m)).astype(np.int32)])
        cols = np.concatenate([c, np.full(m, n // 2, np.int32), (splitmix64(9421 + case, 600) % np.uint64(n)).astype(np.int32)])
        L = am.approx_gemm_chunks(tA, tB, m, n, k, 1, 0, rows, cols)
    finally:
        os.environ.pop("APPROX_KERNEL_SHAPE", None)
    F = oracle.gemm_f32_at(A, B, t, M, rows, cols, np.maximum(L, 1), transA=bool(tA), transB=bool(tB),
                           threads=oracle.default_threads())
    same_bits(C.cpu().numpy()[rows, cols], F, what=f"shape {shape} {name} {CASES[case]}", zero_sign=True)


CONV_GEOMS = [
    # (N, H, W, C, K, R, S, stride, pad)
    (2, 9, 11, 5, 7, 3, 3, (1, 1), (1, 1)),
    (3, 16, 16, 8, 12, 3, 3, (2, 2), (1, 0)),
]


@pytest.mark.parametrize("shape", ["0", "1", "2"])
@pytest.mark.parametrize("name", ["mitchell7", "perturbed8"])
@pytest.mark.parametrize("g", range(len(CONV_GEOMS)))
def test_forced_shape_conv_passes(am, shape, name, g):
    """The convolution's three passes with a shape forced (the weight
    gradient's gather mode ignores shape 2 and keeps its own choice): every
    output the oracle's FP32 sums in the reported order, bit for bit."""
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    N, H, W, C, K, R, S, st, pd = geom = CONV_GEOMS[g]
    P, Q = oracle.conv_out_hw(H, W, R, S, st, pd)
    x = normal(9440 + g, (N, H, W, C))
    w = normal(9441 + g, (R, S, C, K))
    dy = normal(9442 + g, (N, P, Q, K))
    print(f"shape {shape} {name} conv {geom}", flush=True)
    os.environ["APPROX_KERNEL_SHAPE"] = shape
    try:
        outs = {"fwd": (am.conv2d_fwd(dev(x), dev(w), st, pd), x, w),
                "dgrad": (am.conv2d_dgrad(dev(dy), dev(w), x.shape, st, pd), dy, w),
                "wgrad": (am.conv2d_wgrad(dev(x), dev(dy), w.shape, st, pd), x, dy)}
        torch.cuda.synchronize()
        chunks = {}
        for pname, (got, _, _) in outs.items():
            idx = np.arange(got.numel(), dtype=np.int64)
            chunks[pname] = (idx, am.approx_conv2d_chunks(pname, N, H, W, C, K, R, S, st, pd, idx))
    finally:
        os.environ.pop("APPROX_KERNEL_SHAPE", None)
    for pname, (got, t1, t2) in outs.items():
        idx, L = chunks[pname]
        F = oracle.conv2d_f32(pname, t1, t2, geom, t, M, L, idx=idx, threads=oracle.default_threads())
        same_bits(got.cpu().numpy(), F, what=f"shape {shape} {name} conv {geom} {pname}", zero_sign=True)
