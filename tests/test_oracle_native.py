"""Pins of the oracle's native multiplier ("ApproxTrain", arXiv 2209.04161,
Section V: the simulator can call the hardware multiplication in place of the
table; Fig. 6 times the two against each other). The native product is the
exact product of the two floats, so:
  - each product must equal the exact rational product (Python fractions);
  - GEMM sums of small integers must equal integer matrix products exactly;
  - GEMM and Conv2D sums of random data must equal float64 library results
    to the rounding of a different summation order;
  - IEEE special cases (Inf x 0, NaN, subnormal operands) behave as IEEE-754.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from datagen import normal, uniform

from test_oracle_gemm_conv import GEOMS, _torch_conv_ref, close_to


def _floats():
    vals = [1.0, -1.0, 3.0, 0.1, -7.25e-3, 1.5e30, -2.0e-30, 3.4028234663852886e38,
            1.1754943508222875e-38, 1.401298464324817e-45, -5.877471754111438e-39]
    vals += list(normal(501, 40).astype(np.float64))
    vals += list((uniform(502, 20, -1.0, 1.0) * np.float32(1e-20)).astype(np.float64))
    return np.array(vals, dtype=np.float32)


def test_native_product_is_the_exact_rational_product():
    a = _floats()
    b = a[::-1].copy()
    got = oracle.mul_native(a, b)
    for x, y, g in zip(a, b, got):
        assert Fraction(float(x)) * Fraction(float(y)) == Fraction(float(g)), (x, y, g)


def test_native_product_special_values():
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    a = np.array([inf, inf, -inf, 0.0, nan, 2.0, -0.0], np.float32)
    b = np.array([0.0, -3.0, -inf, 5.0, 1.0, nan, 4.0], np.float32)
    got = oracle.mul_native(a, b)
    assert math.isnan(got[0])                              # Inf x 0
    assert got[1] == -math.inf and got[2] == math.inf
    assert got[3] == 0.0 and math.copysign(1.0, got[3]) == 1.0
    assert math.isnan(got[4]) and math.isnan(got[5])
    assert got[6] == 0.0 and math.copysign(1.0, got[6]) == -1.0


@pytest.mark.parametrize("transA,transB", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_native_gemm_of_integers_is_exact(transA, transB):
    m, n, k = 9, 7, 13
    rng = np.random.default_rng(7)
    A = rng.integers(-50, 51, size=(k, m) if transA else (m, k))
    B = rng.integers(-50, 51, size=(n, k) if transB else (k, n))
    R, S = oracle.gemm(A.astype(np.float32), B.astype(np.float32), None, 0,
                       transA=bool(transA), transB=bool(transB))
    opA = (A.T if transA else A).tolist()
    opB = (B.T if transB else B).tolist()
    for i in range(m):
        for j in range(n):
            exact = sum(opA[i][p] * opB[p][j] for p in range(k))
            mag = sum(abs(opA[i][p] * opB[p][j]) for p in range(k))
            assert R[i, j] == exact and S[i, j] == mag


@pytest.mark.parametrize("m,n,k", [(5, 3, 4), (33, 17, 64), (3, 70, 129)])
def test_native_gemm_equals_float64_matmul(m, n, k):
    A = normal(511, (m, k))
    B = normal(512, (k, n))
    R, S = oracle.gemm(A, B, None, 0)
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    close_to(R, A64 @ B64, S)
    close_to(S, np.abs(A64) @ np.abs(B64), S)


def test_native_gemm_keeps_subnormal_and_special_results():
    tiny = np.float32(2.0 ** -70)
    R, _ = oracle.gemm(np.array([[tiny]], np.float32), np.array([[tiny]], np.float32), None, 0)
    assert R[0, 0] == 2.0 ** -140                           # a float32 subnormal sum, kept exact
    A = np.array([[np.inf, 1.0], [np.nan, 0.0]], np.float32)
    B = np.array([[0.0, 2.0], [3.0, 1.0]], np.float32)
    R, _ = oracle.gemm(A, B, None, 0)
    assert math.isnan(R[0, 0]) and R[0, 1] == math.inf
    assert math.isnan(R[1, 0]) and math.isnan(R[1, 1])


@pytest.mark.parametrize("geom", GEOMS)
def test_native_conv_equals_torch_float64(geom):
    N, H, W, C, K, R, S, stride, pad = geom
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(521, (N, H, W, C))
    w = normal(522, (R, S, C, K))
    dy = normal(523, (N, P, Q, K))
    y_ref, dx_ref, dw_ref = _torch_conv_ref(x, w, dy, stride, pad)
    Y, YS = oracle.conv2d_fwd(x, w, None, 0, stride, pad)
    close_to(Y, y_ref, YS)
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, None, 0, stride, pad)
    close_to(DX, dx_ref, DXS)
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, None, 0, stride, pad)
    close_to(DW, dw_ref, DWS)
