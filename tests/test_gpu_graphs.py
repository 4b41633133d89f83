"""Library calls captured into a HIP graph (torch.cuda.CUDAGraph on ROCm).

Once a stream's scratch arena is large enough (a first call on that stream
sizes it), a call queues only kernel launches: the decode, the M = 8 copy
choice, the GEMM kernel (which resets the exponent statistics for the next
call itself) and the split reduction. Such calls can be captured and
replayed. Each replay must give the bits of the eager call; eager work and
synchronisations run between the replays, and every replay is checked.
"""
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


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8"])
def test_captured_calls_replay_the_eager_bits(am, name):
    M, t = TABLES[name]()
    am.approx_lut_load(t, M)
    # a split GEMM (few tiles, long reduction), a whole-tile GEMM and a conv
    A1, B1 = normal(1301, (96, 3000)), normal(1302, (3000, 80))
    A2, B2 = normal(1303, (700, 200)), normal(1304, (200, 300))
    x, w = normal(1305, (2, 12, 12, 8)), normal(1306, (3, 3, 8, 16))
    dA1, dB1, dA2, dB2, dx, dw = (dev(v) for v in (A1, B1, A2, B2, x, w))
    C1 = torch.empty((96, 80), dtype=torch.float32, device="cuda")
    C2 = torch.empty((700, 300), dtype=torch.float32, device="cuda")
    Y = torch.empty((2, 12, 12, 16), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()

    def calls():
        am.approx_gemm(0, 0, 96, 80, 3000, dA1, 3000, dB1, 80, C1, 80, stream=s)
        am.approx_gemm(0, 1, 700, 300, 200, dA2, 200, dev_bt, 200, C2, 300, stream=s)
        am.approx_conv2d_fwd(2, 12, 12, 8, 16, 3, 3, (1, 1), (1, 1), dx, dw, Y, stream=s)

    dev_bt = dev(np.ascontiguousarray(B2.T))
    with torch.cuda.stream(s):
        calls()                                  # eager: sizes the stream's arena
    torch.cuda.synchronize()
    eager = [C1.cpu().numpy().copy(), C2.cpu().numpy().copy(), Y.cpu().numpy().copy()]
    # the eager results against the oracle
    R, S = oracle.gemm(A1, B1, t, M)
    gate(eager[0], R, S, what="eager split gemm")
    R, S = oracle.gemm(A2, B2, t, M)
    gate(eager[1], R, S, what="eager gemm")
    R, S = oracle.conv2d_fwd(x, w, t, M, (1, 1), (1, 1))
    gate(eager[2], R, S, what="eager conv")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    for rep in range(3):
        for out in (C1, C2, Y):
            out.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [C1.cpu().numpy(), C2.cpu().numpy(), Y.cpu().numpy()]
        for i in range(3):
            assert np.array_equal(got[i].view(np.uint32), eager[i].view(np.uint32)), f"replay {rep}, output {i}"
        # eager work between the replays, on the same stream and arena
        with torch.cuda.stream(s):
            calls()
        torch.cuda.synchronize()
        assert np.array_equal(C1.cpu().numpy().view(np.uint32), eager[0].view(np.uint32))


def test_graph_survives_arena_growth_and_table_reload(am):
    """A graph captured on a stream keeps the arena memory and the table it
    captured: a later, larger eager call on the same stream grows the arena
    and another table is loaded, yet every replay still gives the bits of the
    eager call made before the capture (the superseded arena and table are
    kept until approx_release)."""
    M, t = TABLES["perturbed8"]()
    am.approx_lut_load(t, M)
    A, B = normal(1311, (300, 500)), normal(1312, (500, 200))
    dA, dB = dev(A), dev(B)
    C = torch.empty((300, 200), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        am.approx_gemm(0, 0, 300, 200, 500, dA, 500, dB, 200, C, 200, stream=s)
    torch.cuda.synchronize()
    eager = C.cpu().numpy().copy()
    R, S = oracle.gemm(A, B, t, M)
    gate(eager, R, S, what="eager before capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        am.approx_gemm(0, 0, 300, 200, 500, dA, 500, dB, 200, C, 200, stream=s)
    # a call of 16x the scratch on the same stream, then another table
    A3, B3 = dev(normal(1313, (1200, 2000))), dev(normal(1314, (2000, 800)))
    C3 = torch.empty((1200, 800), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        am.approx_gemm(0, 0, 1200, 800, 2000, A3, 2000, B3, 800, C3, 800, stream=s)
    am.approx_lut_load(oracle.lut_generate(7, "mitchell"), 7)
    for rep in range(3):
        C.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().view(np.uint32), eager.view(np.uint32)), f"replay {rep}"
        with torch.cuda.stream(s):          # eager work with the new table between replays
            am.approx_gemm(0, 0, 1200, 800, 2000, A3, 2000, B3, 800, C3, 800, stream=s)
        torch.cuda.synchronize()
