"""approx_gemm_grouped: independent GEMMs sharing one decode launch and one
GEMM-kernel launch. Each member must come out with exactly the bits that an
approx_gemm call of its own gives (same products, same summation order), for
any mix of shapes (split and whole tiles, transposes, members the library
runs in other kernels), with each member's own exponent statistics deciding
its path; the grouped results also pass the oracle's gate. Argument errors
queue nothing.
"""
import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one, splitmix64
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


TABLES = {
    "mitchell7": lambda: (oracle.lut_generate(7, "mitchell"), 7),
    "perturbed8": lambda: (oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16)), 8),
    "arbitrary10": lambda: ((splitmix64(7010, 1 << 20) >> np.uint64(48)).astype(np.uint16), 10),
    "native": lambda: (None, 0),
}


def use(am, name):
    t, M = TABLES[name]()
    if t is None:
        am.approx_native_load()
    else:
        am.approx_lut_load(t, M)
    return t, M


def member(seed, tA, tB, m, n, k, scale=1.0):
    """A member's operands (host), stored as op(A) / op(B) with the flags."""
    A = normal(seed, (k, m) if tA else (m, k)) * np.float32(scale)
    B = normal(seed + 1, (n, k) if tB else (k, n))
    return tA, tB, m, n, k, A.astype(np.float32), B.astype(np.float32)


def calls_of(members):
    out = []
    for (tA, tB, m, n, k, A, B) in members:
        C = torch.full((m, n), -7.0, dtype=torch.float32, device="cuda")
        out.append((tA, tB, m, n, k, dev(A), max(1, A.shape[1]), dev(B), max(1, B.shape[1]), C, n))
    return out


def run_individually(am, members):
    res = []
    for c in calls_of(members):
        am.approx_gemm(*c)
        res.append(host(c[9]).copy())
    return res


def run_grouped(am, members):
    cs = calls_of(members)
    am.approx_gemm_grouped(cs)
    return [host(c[9]).copy() for c in cs]


def same_bits(a, b, what):
    assert a.shape == b.shape, what
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
        f"{what}: {np.count_nonzero(a.view(np.uint32) != b.view(np.uint32))} outputs differ"


MIXES = {
    # a dense layer's backward pair (input and weight gradients), as the MLP workload
    "mlp_pair": [(0, 1, 256, 1024, 1024), (1, 0, 1024, 1024, 256)],
    # split tails, whole tiles, all four transposes, a ragged edge
    "four": [(0, 0, 300, 200, 517), (1, 1, 130, 260, 64), (0, 1, 1000, 129, 96), (1, 0, 77, 390, 1200)],
    # one long member with many tiles beside short ones
    "lopsided": [(0, 0, 1536, 1024, 256), (0, 0, 256, 10, 1024), (1, 0, 1024, 10, 256)],
}


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8", "arbitrary10", "native"])
@pytest.mark.parametrize("mix", sorted(MIXES))
def test_grouped_gives_each_members_own_bits(am, name, mix):
    use(am, name)
    members = [member(9100 + 17 * i + len(mix), *shape) for i, shape in enumerate(MIXES[mix])]
    want = run_individually(am, members)
    got = run_grouped(am, members)
    for i in range(len(members)):
        same_bits(got[i], want[i], f"{name} {mix} member {i} {MIXES[mix][i]}")
    # and again: the first grouped call left every member's stats reset
    got2 = run_grouped(am, members)
    for i in range(len(members)):
        same_bits(got2[i], want[i], f"{name} {mix} member {i}, second call")


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8"])
def test_grouped_parity_with_the_oracle(am, name):
    t, M = use(am, name)
    members = [member(9300, 0, 1, 96, 200, 300), member(9302, 1, 0, 150, 80, 260)]
    got = run_grouped(am, members)
    for i, (tA, tB, m, n, k, A, B) in enumerate(members):
        R, S = oracle.gemm(A, B, t, M, transA=bool(tA), transB=bool(tB))
        gate(got[i], R, S, what=f"grouped {name} member {i}")


def test_grouped_members_run_elsewhere(am):
    """Members that approx_gemm runs in the row-vector kernel, with k = 0, or
    with m = 0 sit beside GEMM-kernel members; every one gets its own bits."""
    use(am, "mitchell7")
    shapes = [(0, 0, 3, 700, 900), (0, 1, 300, 256, 513), (0, 0, 50, 60, 0), (1, 0, 120, 500, 300)]
    members = [member(9400 + i, *s) for i, s in enumerate(shapes)]
    want = run_individually(am, members)
    got = run_grouped(am, members)
    for i in range(len(members)):
        same_bits(got[i], want[i], f"member {i} {shapes[i]}")
    assert np.all(got[2] == 0.0)
    empty = torch.full((0, 5), 1.0, dtype=torch.float32, device="cuda")
    a, b = dev(np.zeros((0, 4), np.float32)), dev(np.zeros((4, 5), np.float32))
    am.approx_gemm_grouped([(0, 0, 0, 5, 4, a, 4, b, 5, empty, 5)])


def test_grouped_members_keep_their_own_exponent_statistics(am):
    """Member 0's operands can overflow (huge op(A) against a huge B: the
    checked path), member 1's cannot (fast path): each member's bits equal
    its own call's, and the oracle's exactly where the order is fixed by a
    single chunk."""
    t, M = use(am, "perturbed8")
    big = member(9500, 0, 0, 200, 130, 96, scale=2.0 ** 100)
    big[6][:] *= np.float32(2.0 ** 60)
    small = member(9502, 0, 0, 260, 140, 96)
    want = run_individually(am, [big, small])
    got = run_grouped(am, [big, small])
    same_bits(got[0], want[0], "overflow-capable member")
    same_bits(got[1], want[1], "ordinary member")
    # products of 2^160 overflow to +-Inf; sums of both signs become NaN
    assert not np.isfinite(got[0]).all(), "the planted magnitudes should overflow some products"
    assert np.isfinite(got[1]).all()
    # an ordinary call after the group: the stats the group left are reset
    again = run_individually(am, [small])
    same_bits(again[0], want[1], "ordinary call after the group")


def test_grouped_call_replays_in_a_graph(am):
    use(am, "mitchell7")
    members = [member(9600, 0, 1, 256, 512, 700), member(9602, 1, 0, 512, 512, 256)]
    want = run_individually(am, members)
    cs = calls_of(members)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        am.approx_gemm_grouped(cs, stream=s)           # eager: sizes the stream's arena
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        am.approx_gemm_grouped(cs, stream=s)
    for rep in range(3):
        for c in cs:
            c[9].fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, c in enumerate(cs):
            same_bits(host(c[9]), want[i], f"replay {rep} member {i}")
        with torch.cuda.stream(s):
            am.approx_gemm_grouped(cs, stream=s)       # eager work between replays
        torch.cuda.synchronize()


def test_grouped_argument_errors_queue_nothing(am):
    use(am, "mitchell7")
    members = [member(9700, 0, 0, 64, 64, 64), member(9702, 0, 0, 64, 64, 64)]
    cs = calls_of(members)
    with pytest.raises(am.ApproxError) as e:
        am.approx_gemm_grouped([])
    assert e.value.status == am.APPROX_EINVAL
    with pytest.raises(am.ApproxError) as e:
        am.approx_gemm_grouped(cs * 3)
    assert e.value.status == am.APPROX_EINVAL
    bad = list(cs[1])
    bad[6] = 10                                        # lda below k
    with pytest.raises(am.ApproxError) as e:
        am.approx_gemm_grouped([cs[0], tuple(bad)])
    assert e.value.status == am.APPROX_EINVAL
    for c in cs:                                       # nothing ran: the fill value is intact
        assert np.all(host(c[9]) == -7.0)
