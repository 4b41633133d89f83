"""GPU parity of the M = 8 table's second copies: the decode pass moves some
lane operands of every 32-row group to the second copy of their table row
(only where that lowers the group's largest LDS bank load). Any copy holds
the same entry, so products stay bit-exact and sums meet the gate; these
cases use random mantissas (so that copies are chosen), every layout that
reads the copies (dense, batched, the three Conv2D images) and an
arbitrary-entry table (so that a row read from the wrong copy or half would
show)."""
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
    return m


def arbitrary_table8():
    """4^8 entries of arbitrary 16-bit values (seeded), none zero."""
    r = splitmix64(0xA8B1, 1 << 16)
    return ((r >> np.uint64(17)) % np.uint64(0xFFFF) + np.uint64(1)).astype(np.uint16)


TABLES = {
    "perturbed8": lambda: oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16)),
    "arbitrary8": arbitrary_table8,
}


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("name", sorted(TABLES))
def test_random_mantissa_products_bit_exact(am, name):
    """C = a b^T with k = 1 over 4096 random rows (groups of 32 random
    mantissas, some zero / Inf / NaN) and 96 columns."""
    t = TABLES[name]()
    am.approx_lut_load(t, 8)
    a = normal(801, (4096,)).view(np.uint32).copy()
    sp = special_values().view(np.uint32)
    a[::97] = sp[np.arange(a[::97].size) % sp.size]
    b = normal(802, (96,)).view(np.uint32)
    C = torch.empty((a.size, b.size), dtype=torch.float32, device="cuda")
    print(f"m8 copies products {name}", flush=True)
    am.approx_gemm(0, 0, a.size, b.size, 1, dev(a.view(np.float32).reshape(-1, 1)), 1,
                   dev(b.view(np.float32).reshape(1, -1)), b.size, C, b.size)
    got = host(C).view(np.uint32)
    want = oracle.amsim_bits(np.repeat(a, b.size), np.tile(b, a.size), t, 8).reshape(a.size, b.size)
    want = np.where(want == 0x80000000, 0, want).astype(np.uint32)
    gnan = np.isnan(got.view(np.float32))
    assert np.array_equal(gnan, np.isnan(want.view(np.float32)))
    assert np.count_nonzero(got[~gnan] != want[~gnan]) == 0


def test_dense_transposed_and_batched(am):
    t = TABLES["arbitrary8"]()
    am.approx_lut_load(t, 8)
    for (m, n, k, ta) in ((300, 70, 90, 0), (130, 40, 77, 1)):
        A = normal(810 + m, (k, m) if ta else (m, k))
        B = normal(811 + m, (k, n))
        R, S = oracle.gemm(A, B, t, 8, transA=bool(ta))
        gate(host(am.gemm(dev(A), dev(B), transA=bool(ta))), R, S, what=f"dense {m}x{n}x{k} tA={ta}")
    m, n, k, nb = 96, 33, 50, 3
    A = normal(820, (nb, m, k))
    B = normal(821, (nb, k, n))
    C = torch.empty((nb, m, n), dtype=torch.float32, device="cuda")
    am.approx_gemm_strided_batched(0, 0, m, n, k, dev(A), k, m * k, dev(B), n, k * n, C, n, m * n, nb)
    got = host(C)
    for i in range(nb):
        R, S = oracle.gemm(A[i], B[i], t, 8)
        gate(got[i], R, S, what=f"batch {i}")


@pytest.mark.parametrize("geom", [
    (2, 8, 33, 6, 5, 3, 3, (1, 1), (1, 1)),
    (1, 9, 40, 3, 4, 3, 3, (2, 2), (1, 1)),
    (1, 6, 12, 40, 7, 2, 3, (1, 1), (0, 1)),
])
def test_conv_images(am, geom):
    N, H, W, C, K, R, S, stride, pad = geom
    t = TABLES["arbitrary8"]()
    am.approx_lut_load(t, 8)
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(831, (N, H, W, C))
    w = normal(832, (R, S, C, K))
    dy = normal(833, (N, P, Q, K))
    print(f"m8 conv {geom}", flush=True)
    Y, YS = oracle.conv2d_fwd(x, w, t, 8, stride, pad)
    gate(host(am.conv2d_fwd(dev(x), dev(w), stride, pad)), Y, YS, what="fwd")
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, t, 8, stride, pad)
    gate(host(am.conv2d_dgrad(dev(dy), dev(w), x.shape, stride, pad)), DX, DXS, what="dgrad")
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, t, 8, stride, pad)
    gate(host(am.conv2d_wgrad(dev(x), dev(dy), w.shape, stride, pad)), DW, DWS, what="wgrad")
