"""approx_gemm_noalloc: the allocation-free variant of approx_gemm.

Its scratch is one fixed array per device, so it must give approx_gemm's bits
(same kernels, same plan) call after call, whatever the previous call left in
that array: two calls in a row, the second smaller; the row-vector path; a
table with second copies (M = 8); a HIP graph replay; and a call too large
for the array, refused before anything is written.
"""
import ctypes

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one
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


TABLES = {
    "mitchell7": lambda: (7, oracle.lut_generate(7, "mitchell")),
    "perturbed8": lambda: (8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16))),
}


def both(am, m, n, k, A, B, seed_out):
    """C from approx_gemm and from approx_gemm_noalloc (through the C ABI),
    each into an output prefilled with a different value."""
    dA, dB = dev(A), dev(B)
    C0 = torch.full((m, n), 3.0, dtype=torch.float32, device="cuda")
    C1 = torch.full((m, n), -7.0, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    L = am.lib()
    assert L.approx_gemm(0, 0, m, n, k, dA.data_ptr(), k, dB.data_ptr(), n, C0.data_ptr(), n, s) == am.APPROX_OK
    assert L.approx_gemm_noalloc(0, 0, m, n, k, dA.data_ptr(), k, dB.data_ptr(), n, C1.data_ptr(), n, s) == am.APPROX_OK
    torch.cuda.synchronize()
    return C0.cpu().numpy(), C1.cpu().numpy()


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8"])
def test_noalloc_matches_approx_gemm_two_calls(am, name):
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    # first a larger call (GEMM kernel, split reduction), then a smaller one
    # (GEMM kernel, whole tiles), then a row-vector call with split partials
    for (m, n, k) in ((300, 200, 3000), (100, 50, 400), (16, 300, 5000)):
        print(f"noalloc {name} {m}x{n}x{k}", flush=True)
        A = normal(1400 + m, (m, k))
        B = normal(1401 + n, (k, n))
        ref, got = both(am, m, n, k, A, B, m)
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), (m, n, k)
        R, S = oracle.gemm(A, B, t, M)
        gate(got, R, S, what=f"noalloc {m}x{n}x{k}")


def test_noalloc_graph_replay(am):
    """Captured into a HIP graph: the replays give the eager bits, with
    eager allocation-free calls of another size between them."""
    M, t = TABLES["perturbed8"]()
    am.approx_lut_load(t, M)
    A, B = normal(1411, (260, 700)), normal(1412, (700, 90))
    dA, dB = dev(A), dev(B)
    C = torch.empty((260, 90), dtype=torch.float32, device="cuda")
    A2, B2 = dev(normal(1413, (400, 300))), dev(normal(1414, (300, 500)))
    C2 = torch.empty((400, 500), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        am.approx_gemm_noalloc(0, 0, 260, 90, 700, dA, 700, dB, 90, C, 90, stream=s)
    torch.cuda.synchronize()
    eager = C.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        am.approx_gemm_noalloc(0, 0, 260, 90, 700, dA, 700, dB, 90, C, 90, stream=s)
    for rep in range(3):
        C.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().view(np.uint32), eager.view(np.uint32)), f"replay {rep}"
        with torch.cuda.stream(s):
            am.approx_gemm_noalloc(0, 0, 400, 500, 300, A2, 300, B2, 500, C2, 500, stream=s)
        torch.cuda.synchronize()
    R, S = oracle.gemm(A, B, t, M)
    gate(eager, R, S, what="noalloc graph")


def test_noalloc_refuses_oversized_call(am):
    """A call whose decoded operands exceed the fixed scratch returns
    APPROX_ESCRATCH before queuing anything: C keeps its contents."""
    M, t = TABLES["mitchell7"]()
    am.approx_lut_load(t, M)
    cap = am.approx_gemm_noalloc_max_bytes()
    assert cap > 0
    # 8 bytes per decoded element (a table is loaded): (m + n) * k * 8 > cap
    m = n = 2048
    k = int(cap // (8 * (m + n))) + 64
    A = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    B = torch.zeros((k, n), dtype=torch.float32, device="cuda")
    C = torch.full((m, n), 9.0, dtype=torch.float32, device="cuda")
    rc = am.lib().approx_gemm_noalloc(0, 0, m, n, k, A.data_ptr(), k, B.data_ptr(), n, C.data_ptr(), n,
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == am.APPROX_ESCRATCH
    assert "scratch" in am.approx_status_string(rc)
    torch.cuda.synchronize()
    assert bool((C == 9.0).all())
