"""Pins of the oracle's FP32-order sums (reading R20: chunks of L positions,
each summed from +0 in ascending order, then the chunk sums from +0; every
addition rounded to nearest even, a fused multiply-add per step for the
native multiplier).

- hand-worked sums (tests/golden/fp32_order.txt): ties to even, chunking,
  overflow to infinity and to NaN, order dependence, the fused native step;
- numpy's sequential float32 accumulation (np.add.accumulate, a library
  routine) over the oracle's pinned products, chunk by chunk;
- sums that are exact in FP32 equal the double-precision oracle;
- Conv2D: the implicit sums in the documented sequences equal the GEMM
  FP32-order sums over explicit IM2COL matrices laid out in that order.
"""
import os

import numpy as np
import pytest

import oracle
from datagen import normal
from test_oracle_gemm_conv import GEOMS, _im2col

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_cases():
    cases = []
    with open(os.path.join(GOLDEN, "fp32_order.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            head, a, b = (part.split() for part in line.split(";"))
            name, mult, L, want = head
            cases.append((name, mult, int(L), float.fromhex(want) if want not in ("inf", "nan") else float(want),
                          [float.fromhex(v) if "x" in v else float(v) for v in a],
                          [float.fromhex(v) if "x" in v else float(v) for v in b]))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_hand_worked_sums(case):
    name, mult, L, want, a, b = case
    A = np.array([a], np.float32)                 # 1 x k
    B = np.array(b, np.float32).reshape(-1, 1)    # k x 1
    assert np.array_equal(A.astype(np.float64).ravel(), a) and np.array_equal(B.astype(np.float64).ravel(), b)
    lut, M = (oracle.lut_generate(7, "exact"), 7) if mult == "exact7" else (None, 0)
    got = oracle.gemm_f32_at(A, B, lut, M, [0], [0], L)[0]
    if np.isnan(want):
        assert np.isnan(got), name
    else:
        assert got == np.float32(want), (name, got.hex() if hasattr(got, "hex") else got, want)


def _accumulate(products, L):
    """np.add.accumulate in float32: sequential sums from +0, chunk by chunk."""
    p = np.asarray(products, np.float32)
    chunk_sums = []
    for c0 in range(0, p.size, L):
        chunk_sums.append(np.add.accumulate(np.concatenate([np.float32([0.0]), p[c0:c0 + L]]))[-1])
    return np.add.accumulate(np.concatenate([np.float32([0.0]), np.array(chunk_sums, np.float32)]))[-1]


@pytest.mark.parametrize("name", ["mitchell7", "perturbed8", "arbitrary5"])
@pytest.mark.parametrize("k,L", [(1, 1), (37, 37), (37, 1000), (100, 7), (100, 12), (257, 64), (64, 1)])
def test_gemm_f32_equals_numpy_sequential_sums(name, k, L):
    from datagen import PERTURB_SEED, pm_one, splitmix64
    if name == "mitchell7":
        M, lut = 7, oracle.lut_generate(7, "mitchell")
    elif name == "perturbed8":
        M, lut = 8, oracle.lut_perturb(8, oracle.lut_generate(8, "exact"), pm_one(PERTURB_SEED, 1 << 16))
    else:
        M, lut = 5, (splitmix64(7305, 1 << 10) >> np.uint64(48)).astype(np.uint16)
    A = normal(900 + k, (3, k), std=4.0)
    B = normal(901 + L, (k, 4))
    got = oracle.gemm_f32(A, B, lut, M, L)
    for i in range(3):
        for j in range(4):
            prods = oracle.amsim(A[i], B[:, j], lut, M)
            want = _accumulate(prods, L)
            assert got[i, j].view(np.uint32) == np.float32(want).view(np.uint32), (i, j)


def test_native_f32_equals_numpy_when_products_are_exact():
    """Operands of at most 12 significant bits: every native product is exact
    in FP32, so a fused step rounds like an FP32 addition of the product."""
    k = 150
    A = np.round(normal(911, (2, k), std=64.0)).astype(np.float32)     # integers below 2^12
    B = (np.round(normal(912, (k, 3), std=64.0)) / 64.0).astype(np.float32)
    for L in (k, 16, 1):
        got = oracle.gemm_f32(A, B, None, 0, L)
        for i in range(2):
            for j in range(3):
                prods = A[i].astype(np.float64) * B[:, j].astype(np.float64)
                assert np.all(prods.astype(np.float32).astype(np.float64) == prods)
                assert got[i, j] == _accumulate(prods.astype(np.float32), L)


def test_exact_sums_equal_the_double_oracle():
    """Small integer products: every FP32 partial sum is exact, so any order
    gives the double-precision oracle's sum."""
    M, lut = 7, oracle.lut_generate(7, "exact")
    A = np.round(normal(921, (5, 200), std=8.0)).astype(np.float32)
    B = np.round(normal(922, (200, 6), std=8.0)).astype(np.float32)
    R, _ = oracle.gemm(A, B, lut, M)
    for L in (1, 8, 200):
        assert np.array_equal(oracle.gemm_f32(A, B, lut, M, L).astype(np.float64), R)


def test_threaded_driver_gives_the_same_bits():
    M, lut = 7, oracle.lut_generate(7, "mitchell")
    A, B = normal(931, (40, 300)), normal(932, (300, 30))
    rows, cols = np.meshgrid(np.arange(40), np.arange(30), indexing="ij")
    one = oracle.gemm_f32_at(A, B, lut, M, rows.ravel(), cols.ravel(), 64)
    many = oracle.gemm_f32_at(A, B, lut, M, rows.ravel(), cols.ravel(), 64, threads=4)
    assert np.array_equal(one.view(np.uint32), many.view(np.uint32))


def _pad_channels(cols, R, S, C, C4):
    """IM2COL columns (r, s, c) -> (r, s, c') with c' < C4, zero past C."""
    out = np.zeros((cols.shape[0], R, S, C4), np.float32)
    out[:, :, :, :C] = cols.reshape(-1, R, S, C)
    return out.reshape(cols.shape[0], R * S * C4)


@pytest.mark.parametrize("geom", GEOMS)
@pytest.mark.parametrize("L", [4, 8, 1 << 20])
def test_conv_f32_sequences_equal_explicit_im2col(geom, L):
    """Same products, same positions: the implicit FP32-order sums equal the
    GEMM FP32-order sums over explicit IM2COL matrices whose columns follow
    the documented sequence (channels padded to a multiple of 4 with zeros,
    whose products change no sum)."""
    N, H, W, C, K, R, S, stride, pad = geom
    M, lut = 7, oracle.lut_generate(7, "mitchell")
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(941, (N, H, W, C))
    w = normal(942, (R, S, C, K))
    dy = normal(943, (N, P, Q, K))
    g = (N, H, W, C, K, R, S, stride, pad)
    C4, K4 = (C + 3) // 4 * 4, (K + 3) // 4 * 4
    # forward: columns (r, s, c'), weights rows (r, s, c')
    cols = _pad_channels(_im2col(x, R, S, stride, pad), R, S, C, C4)
    wp = np.zeros((R, S, C4, K), np.float32)
    wp[:, :, :C, :] = w
    want = oracle.gemm_f32(cols, wp.reshape(R * S * C4, K), lut, M, L)
    got = oracle.conv2d_f32("fwd", x, w, g, lut, M, L)
    assert np.array_equal(got.view(np.uint32), want.ravel().view(np.uint32))
    # weight gradient: IM2COL(x)^T over (n, p, q), then dY
    cols = _im2col(x, R, S, stride, pad)
    want = oracle.gemm_f32(cols, dy.reshape(-1, K), lut, M, L, transA=True)
    got = oracle.conv2d_f32("wgrad", x, dy, g, lut, M, L)
    assert np.array_equal(got.view(np.uint32), want.ravel().view(np.uint32))
    # input gradient: padded, dilated errors, taps in reverse order
    sh, sw = stride
    ph, pw = pad
    Hd, Wd = (P - 1) * sh + 1, (Q - 1) * sw + 1
    dil = np.zeros((N, Hd, Wd, K), np.float32)
    dil[:, ::sh, ::sw, :] = dy
    lo_h, lo_w = R - 1 - ph, S - 1 - pw
    big = np.zeros((N, H + 2 * R + Hd, W + 2 * S + Wd, K), np.float32)
    oh, ow = R + 2, S + 2
    big[:, oh + lo_h: oh + lo_h + Hd, ow + lo_w: ow + lo_w + Wd, :] = dil
    colsd = np.zeros((N, H, W, R, S, K4), np.float32)     # columns (u1, u2, k'), u1 = R-1-r
    wd = np.zeros((R, S, K4, C), np.float32)
    for u1 in range(R):
        for u2 in range(S):
            r, s = R - 1 - u1, S - 1 - u2
            colsd[:, :, :, u1, u2, :K] = big[:, oh + u1: oh + u1 + H, ow + u2: ow + u2 + W, :]
            wd[u1, u2, :K, :] = w[r, s].T
    want = oracle.gemm_f32(colsd.reshape(N * H * W, R * S * K4), wd.reshape(R * S * K4, C), lut, M, L)
    got = oracle.conv2d_f32("dgrad", dy, w, g, lut, M, L)
    assert np.array_equal(got.view(np.uint32), want.ravel().view(np.uint32))
