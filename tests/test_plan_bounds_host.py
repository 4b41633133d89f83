"""Host-side bounds check of the library's plans (no GPU): for every GEMM
and Conv2D case the GPU tests draw (tests/test_gpu_random_cases.py), the five
workloads, and extreme shapes, at table widths 0 (native), 3, 7, 8 and 10,
the largest offset each kernel of the planned call touches must lie inside
the buffer the plan allocates: the decoded panels (decode writes, GEMM-kernel
reads of row bases plus k-step offsets, gather mode's zero region, uniform
rows and columns), the split partials, the M = 8 copy-choice groups, the
table image and the scratch total. The offsets come from the library's
test hook amx_plan_check, which walks them with the kernels' index
formulas."""
import ctypes

import numpy as np
import pytest

from datagen import configs as cfg

SLOTS = ["decode lane", "decode uniform", "read lane", "read uniform", "partials", "copy groups", "table",
         "scratch"]
WIDTHS = [0, 3, 7, 8, 10]


@pytest.fixture(scope="module")
def check():
    import approximate_multiplier_dnn_amd as am
    f = am.lib().amx_plan_check
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int

    def run(kind, args, M):
        a = np.ascontiguousarray(args, dtype=np.int32)
        need = np.zeros(len(SLOTS), np.int64)
        have = np.zeros(len(SLOTS), np.int64)
        rc = f(kind, a.ctypes.data, M, need.ctypes.data, have.ctypes.data)
        assert rc >= 0, (kind, list(args), M, rc)
        bad = [(SLOTS[i], int(need[i]), int(have[i])) for i in range(len(SLOTS)) if need[i] > have[i]]
        assert not bad, (kind, list(args), M, bad)
        assert need[2] > 0 and need[3] > 0, "the check walked no offsets"
        return need, have
    return run


def _gemm_cases():
    from test_gpu_random_cases import GEMM_CASES
    out = [(c["tA"], c["tB"], c["m"], c["n"], c["k"], c["batch"]) for c in GEMM_CASES]
    # the workloads' GEMMs (the row-vector route aside, every shape also through the GEMM kernel)
    out += [(0, 0, 64, 64, 64, 1), (0, 0, 8192, 8192, 8192, 1)]
    out += [(ta, tb, m, n, k, 1) for (_, ta, tb, m, n, k, _, _) in cfg.mlp_gemms()]
    out += [(0, 0, 8192, 2304, 768, 1), (0, 1, 512, 512, 64, 192), (0, 0, 512, 64, 512, 192), (0, 0, 8192, 768, 768, 1)]
    # extremes: one row, one column, k = 1, ragged tiles, tail-split tiles
    out += [(0, 0, 1, 1, 1, 1), (1, 1, 1, 3000, 1, 3), (0, 1, 2049, 17, 5, 2), (1, 0, 133020, 64, 400, 1),
            (0, 0, 257, 129, 4097, 4)]
    return out


def _conv_cases():
    from test_gpu_random_cases import CONV_CASES
    out = [(c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], *c["stride"], *c["pad"]) for c in CONV_CASES]
    s = cfg.CONV_SHAPE
    out.append((s["N"], s["H"], s["W"], s["C"], s["K"], s["R"], s["S"], *s["stride"], *s["pad"]))
    out += [(1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0), (3, 7, 5, 5, 3, 5, 5, 3, 2, 4, 4), (130, 32, 32, 64, 64, 3, 3, 1, 1, 1, 1),
            (2, 33, 9, 3, 70, 3, 1, 2, 3, 1, 0)]
    return out


@pytest.mark.parametrize("M", WIDTHS)
def test_gemm_plans_stay_inside_their_buffers(check, M):
    for args in _gemm_cases():
        check(0, args, M)


@pytest.mark.parametrize("M", WIDTHS)
def test_conv_plans_stay_inside_their_buffers(check, M):
    for args in _conv_cases():
        for kind in (1, 2, 3):
            check(kind, args, M)


def test_check_sees_the_gather_mode_zero_region(check):
    """The weight gradient reads a zero region past the image for reduction
    indices beyond N P Q: the lane reads must reach into it (and stay inside
    the allocation)."""
    need, have = check(3, (1, 5, 5, 3, 2, 3, 3, 1, 1, 1, 1), 7)   # N P Q = 25: indices 25..27 padded
    assert need[2] > 1 * 7 * 7 * 3          # beyond the padded image body
    assert need[2] <= have[2]


def test_check_rejects_invalid_arguments(check):
    import approximate_multiplier_dnn_amd as am
    f = am.lib().amx_plan_check
    need = np.zeros(len(SLOTS), np.int64)
    have = np.zeros(len(SLOTS), np.int64)
    bad = np.array([0, 0, 0, 5, 5, 1], np.int32)
    assert f(0, bad.ctypes.data, 7, need.ctypes.data, have.ctypes.data) == am.APPROX_EINVAL
    assert f(9, bad.ctypes.data, 7, need.ctypes.data, have.ctypes.data) == am.APPROX_EINVAL


def test_row_vector_group_rows_stay_inside_the_item():
    """The row-vector kernel loads B in groups of indices and may request a
    group that starts past the item's last index (the next group, asked for
    ahead of use). Every row a group load reads must lie inside the item
    [k0, k1), offsets from the load's base row must be non-negative (they are
    unsigned 32-bit byte offsets on the GPU), and index kg + g must read row
    kg + g while that is inside the item (else row k1 - 1)."""
    import approximate_multiplier_dnn_amd as am
    f = am.lib().amx_gemv_group_rows
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    rows = np.zeros(8, np.int32)
    for k0 in (0, 3, 64):
        for k1 in range(k0 + 1, k0 + 41):
            for kg in range(k0, k1 + 17):
                for ng in (4, 8):
                    base = f(k1, kg, ng, rows.ctypes.data)
                    got = rows[:ng]
                    assert k0 <= base <= k1 - 1, (k0, k1, kg, ng, base)
                    assert np.all(got >= base) and np.all(got <= k1 - 1), (k0, k1, kg, ng, list(got))
                    want = np.minimum(kg + np.arange(ng), k1 - 1)
                    assert np.array_equal(got, want), (k0, k1, kg, ng, list(got))
    assert f(0, 0, 4, rows.ctypes.data) == -1


@pytest.mark.parametrize("shape", ["0", "1", "2"])
def test_gemm_plans_of_every_forced_shape_stay_inside(check, shape, monkeypatch):
    """The same GEMM cases with each workgroup shape forced
    (APPROX_KERNEL_SHAPE), at a table in LDS and one in global memory."""
    monkeypatch.setenv("APPROX_KERNEL_SHAPE", shape)
    for M in (7, 8, 10):
        for args in _gemm_cases():
            check(0, args, M)


def _plan_info(kind, args, M):
    import approximate_multiplier_dnn_amd as am
    f = am.lib().amx_plan_info
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_longlong
    a = np.zeros(12, np.int32)
    a[:len(args)] = args
    out = np.zeros(12, np.int32)
    items = f(kind, a.ctypes.data, M, out.ctypes.data)
    assert items >= 0, (kind, args, M, items)
    return int(items), out


def test_shape_choice_follows_the_split_model(monkeypatch):
    """Small dense GEMMs (the MLP's) take the 128 x 128 tiles of shape 2 and
    half as many reduction chunks as shape 0 would cut; GEMMs whose 256 x 128
    tiles fill the GPU keep shape 0; the convolution's weight gradient (gather
    mode, which has no shape-2 kernel) never takes shape 2."""
    monkeypatch.delenv("APPROX_KERNEL_SHAPE", raising=False)
    _, o = _plan_info(0, (0, 0, 256, 1024, 1024, 1), 7)
    assert (o[0], o[3], o[4], o[8]) == (2, 128, 128, 16), list(o)
    _, o = _plan_info(0, (1, 0, 1024, 1024, 256, 1), 7)
    assert o[0] == 2, list(o)
    for args in ((0, 0, 8192, 8192, 8192, 1), (0, 0, 4096, 4096, 1024, 1)):
        _, o = _plan_info(0, args, 8)
        assert o[0] == 0, (args, list(o))
    for args in _conv_cases():
        _, o = _plan_info(3, args, 7)
        assert o[0] in (0, 1), (args, list(o))
