"""Fast/checked decisions per k-segment (64 reduction indices). A dense GEMM
whose operands as a whole could leave the format's range (one planted huge or
tiny element) runs the checked path, or the path with underflow, only on the
k-segments whose own exponent ranges need it, and the fast path on the rest.
The paths give the same bits wherever more than one applies, so the result
must equal, bit for bit, both the same call forced onto the checked path and
the oracle's FP32 sums in the library's order. Both operand decodes that
record segments are covered (op(B) copied by rows, and op(B) transposed
through tiles), as are a route that records none (op(A) transposed), split
reductions, the table in global memory (M = 10), and repeated calls and graph
replays (the ranges that earlier calls recorded carry another generation tag
and are never taken as the current call's).
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
    "exact7": lambda: (7, oracle.lut_generate(7, "exact")),
    "perturbed8": lambda: (8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16))),
    "arbitrary10": lambda: (10, (splitmix64(7010, 1 << 20) >> np.uint64(48)).astype(np.uint16)),
}


@pytest.fixture(scope="module")
def am():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import approximate_multiplier_dnn_amd as m
    yield m
    os.environ.pop("APPROX_FORCE_CHECKED", None)
    m.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(x):
    torch.cuda.synchronize()
    return x.cpu().numpy()


def run(am, A, B, tA, tB, m, n, k, forced=False):
    C = torch.full((m, n), -3.0, dtype=torch.float32, device="cuda")
    if forced:
        os.environ["APPROX_FORCE_CHECKED"] = "1"
    try:
        am.approx_gemm(tA, tB, m, n, k, dev(A), A.shape[1], dev(B), B.shape[1], C, n)
        return host(C)
    finally:
        os.environ.pop("APPROX_FORCE_CHECKED", None)


def oracle_bits(am, t, M, A, B, tA, tB, m, n, k, rows, cols):
    L = am.approx_gemm_chunks(tA, tB, m, n, k, 1, 0, rows, cols)
    return oracle.gemm_f32_at(A, B, t, M, rows, cols, np.maximum(L, 1), transA=bool(tA), transB=bool(tB),
                              threads=oracle.default_threads())


def planted(seed, tA, tB, m, n, k, where, value):
    """N(0, 1) operands stored for the flags; op(A)(i, q) or op(B)(q, j) set to
    `value` at index q = where[1] (which == 'A': row where[0]; 'B': column)."""
    A = normal(seed, (k, m) if tA else (m, k))
    B = normal(seed + 1, (n, k) if tB else (k, n))
    which, i, q = where
    if which == "A":
        if tA:
            A[q, i] = value
        else:
            A[i, q] = value
    else:
        if tB:
            B[i, q] = value
        else:
            B[q, i] = value
    return A, B


CASES = [
    # (flags, shape, planted operand/row-or-column/index, value, what it exercises)
    ((0, 0), (300, 256, 2000), ("A", 17, 1234), 2.0 ** 126, "huge op(A): one checked segment; B copied by rows"),
    ((0, 0), (300, 256, 2000), ("B", 200, 70), -(2.0 ** 126), "huge op(B) in segment 1"),
    ((0, 1), (300, 256, 2000), ("B", 5, 1999), 2.0 ** 126, "huge op(B) in the last (partial) segment; B transposed"),
    ((0, 0), (300, 256, 2000), ("A", 3, 640), 2.0 ** -120, "tiny op(A): one segment with underflow"),
    ((0, 0), (96, 80, 3000), ("A", 40, 2047), 2.0 ** 126, "every tile split: the segment crosses no chunk"),
    ((1, 0), (200, 160, 900), ("A", 11, 300), 2.0 ** 126, "op(A) transposed: no segment ranges, whole call checked"),
]


@pytest.mark.parametrize("name", ["exact7", "perturbed8", "arbitrary10"])
@pytest.mark.parametrize("case", range(len(CASES)), ids=[c[4].split(":")[0] for c in CASES])
def test_segment_paths_give_the_checked_bits(am, name, case):
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    (tA, tB), (m, n, k), where, value, what = CASES[case]
    A, B = planted(9800 + case, tA, tB, m, n, k, where, np.float32(value))
    got = run(am, A, B, tA, tB, m, n, k)
    want = run(am, A, B, tA, tB, m, n, k, forced=True)
    same_bits(got, want, what=f"{name} {what}: segments against the forced checked path", zero_sign=True)
    # the oracle on the rows and columns through the planted element, and a sample elsewhere
    which, i, _ = where
    r = np.arange(m, dtype=np.int32)
    c = np.arange(n, dtype=np.int32)
    if which == "A":
        rows = np.concatenate([np.full(n, i, np.int32), (splitmix64(9900 + case, 512) % np.uint64(m)).astype(np.int32)])
        cols = np.concatenate([c, (splitmix64(9901 + case, 512) % np.uint64(n)).astype(np.int32)])
    else:
        rows = np.concatenate([r, (splitmix64(9900 + case, 512) % np.uint64(m)).astype(np.int32)])
        cols = np.concatenate([np.full(m, i, np.int32), (splitmix64(9901 + case, 512) % np.uint64(n)).astype(np.int32)])
    F = oracle_bits(am, t, M, A, B, tA, tB, m, n, k, rows, cols)
    same_bits(got[rows, cols], F, what=f"{name} {what}: against the FP32-order oracle", zero_sign=True)


def test_segment_ranges_reset_between_calls(am):
    """A call with a planted element, then the same shapes with ordinary
    operands, then the planted call again: each gives its forced-checked
    bits (the ranges the first call's decode recorded do not leak into the
    second, whose every segment is fast)."""
    M, t = TABLES["perturbed8"]()
    am.approx_lut_load(t, M)
    m, n, k = 256, 384, 1500
    Ap, Bp = planted(9950, 0, 0, m, n, k, ("A", 100, 777), np.float32(2.0 ** 126))
    Ao, Bo = planted(9952, 0, 0, m, n, k, ("A", 0, 0), np.float32(0.5))
    for rep in range(2):
        for (A, B, what) in ((Ap, Bp, "planted"), (Ao, Bo, "ordinary")):
            got = run(am, A, B, 0, 0, m, n, k)
            want = run(am, A, B, 0, 0, m, n, k, forced=True)
            same_bits(got, want, what=f"{what} call {rep}", zero_sign=True)


def test_segments_under_graph_replay(am):
    """A call captured on ordinary data, eager calls on the same stream in
    between (later generations), then the captured input changed in place to
    hold a planted element: each replay gives the forced-checked bits of the
    data it reads (ranges of other generations are never taken as the
    replay's own)."""
    M, t = TABLES["perturbed8"]()
    am.approx_lut_load(t, M)
    m, n, k = 256, 384, 1500
    A0, B0 = planted(9960, 0, 0, m, n, k, ("A", 0, 0), np.float32(0.5))
    A1 = A0.copy()
    A1[77, 900] = np.float32(2.0 ** 126)
    dA, dB = dev(A0), dev(B0)
    C = torch.empty((m, n), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    call = lambda: am.approx_gemm(0, 0, m, n, k, dA, k, dB, n, C, n, stream=s)
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    want0 = run(am, A0, B0, 0, 0, m, n, k, forced=True)
    want1 = run(am, A1, B0, 0, 0, m, n, k, forced=True)
    for rep, (A, want) in enumerate(((A0, want0), (A1, want1), (A0, want0), (A1, want1))):
        dA.copy_(torch.from_numpy(A))
        with torch.cuda.stream(s):                     # eager calls in between: later generations
            call()
            call()
        torch.cuda.synchronize()
        C.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        same_bits(host(C), want, what=f"replay {rep}", zero_sign=True)
