"""Pins of the oracle's GEMM and Conv2D passes: with the exact table and
M-bit-truncated operands every product is exact, so the sums must equal
float64 library results (numpy matmul, torch conv2d and its autograd
gradients); the implicit conv sums must equal explicit IM2COL + GEMM
(Section VI-B of "ApproxTrain", arXiv 2209.04161); and a hand-worked
Mitchell matrix must come out as worked by hand."""
import os

import numpy as np
import pytest
import torch

import oracle
from datagen import normal, uniform

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def trunc(x, M):
    """DAZ then keep the top M fraction bits (what the table sees)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    e = (b >> 23) & 0xFF
    b = np.where(e == 0, b & 0x80000000, b & np.uint32((0xFFFFFFFF << (23 - M)) & 0xFFFFFFFF))
    return b.astype(np.uint32).view(np.float32)


def close_to(R, ref, S, tol=1e-12):
    """|R - ref| <= tol * S element-wise (both are float64 sums of the same
    exact products in different orders)."""
    R, ref, S = (np.asarray(v, dtype=np.float64) for v in (R, ref, S))
    assert R.shape == ref.shape == S.shape
    assert np.all(np.abs(R - ref) <= tol * S + 1e-300), np.max(np.abs(R - ref) / np.maximum(S, 1e-300))


@pytest.mark.parametrize("transA,transB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("m,n,k", [(7, 5, 3), (33, 17, 64), (64, 64, 64), (3, 70, 129)])
def test_gemm_exact_table_equals_float64_matmul(transA, transB, m, n, k):
    M = 7
    lut = oracle.lut_generate(M, "exact")
    A = normal(1, (k, m) if transA else (m, k))
    B = normal(2, (n, k) if transB else (k, n))
    R, S = oracle.gemm(A, B, lut, M, transA=bool(transA), transB=bool(transB))
    At = trunc(A, M).astype(np.float64)
    Bt = trunc(B, M).astype(np.float64)
    opA = At.T if transA else At
    opB = Bt.T if transB else Bt
    close_to(R, opA @ opB, S)
    close_to(S, np.abs(opA) @ np.abs(opB), S)


def test_gemm_with_leading_dimension_larger_than_columns():
    M = 7
    lut = oracle.lut_generate(M, "mitchell")
    big = normal(3, (20, 40))
    A = big[:, :13]            # 20 x 13 view with lda = 40
    B = normal(4, (13, 9))
    R1, S1 = oracle.gemm(np.ascontiguousarray(A), B, lut, M)
    # the library call path with an explicit lda
    Rf = np.zeros((20, 9))
    Sf = np.zeros((20, 9))
    L = oracle.lib()
    Bc = np.ascontiguousarray(B)
    L.orc_gemm(0, 0, 20, 9, 13, oracle._ptr(big), 40, oracle._ptr(Bc), 9,
               oracle._ptr(lut), M, 8, oracle._ptr(Rf), oracle._ptr(Sf))
    assert np.array_equal(R1, Rf) and np.array_equal(S1, Sf)


def test_hand_worked_matrix():
    vals = {}
    with open(os.path.join(GOLDEN, "hand_matrix_mitchell.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *nums = line.split()
                vals[key] = np.array([float(v) for v in nums]).reshape(2, 2)
    A = vals["A"].astype(np.float32)
    B = vals["B"].astype(np.float32)
    R, _ = oracle.gemm(A, B, oracle.lut_generate(7, "mitchell"), 7)
    assert np.array_equal(R, vals["C_mitchell"])
    R, _ = oracle.gemm(A, B, oracle.lut_generate(7, "exact"), 7)
    assert np.array_equal(R, vals["C_exact"])


def test_mitchell_gemm_equals_sum_of_formula_products():
    """Brute force from Mitchell's formula on the truncated operands."""
    M = 7
    lut = oracle.lut_generate(M, "mitchell")
    A = normal(5, (9, 31))
    B = normal(6, (31, 11))
    R, S = oracle.gemm(A, B, lut, M)

    def parts(x):
        b = trunc(x, M).view(np.uint32).astype(np.int64)
        sgn = np.where(b >> 31, -1.0, 1.0)
        e = ((b >> 23) & 0xFF) - 127
        f = ((b >> (23 - M)) & ((1 << M) - 1)) / float(1 << M)
        return sgn, e, f

    sa, ea, fa = parts(A)
    sb, eb, fb = parts(B)
    s = fa[:, :, None] + fb[None, :, :]
    sig = np.where(s < 1.0, 1.0 + s, 2.0 * s)
    prod = sa[:, :, None] * sb[None, :, :] * sig * np.exp2(ea[:, :, None] + eb[None, :, :])
    close_to(R, prod.sum(axis=1), S)


def test_gemm_k_zero_and_sampled_outputs():
    lut = oracle.lut_generate(7, "mitchell")
    R, S = oracle.gemm(np.zeros((4, 0), np.float32), np.zeros((0, 3), np.float32), lut, 7)
    assert R.shape == (4, 3) and np.all(R == 0) and np.all(S == 0)
    A = normal(7, (40, 50))
    B = normal(8, (50, 30))
    R, S = oracle.gemm(A, B, lut, 7, transB=False)
    rows = np.array([0, 39, 5, 17])
    cols = np.array([29, 0, 5, 11])
    r, s = oracle.gemm_at(A, B, lut, 7, rows, cols)
    assert np.array_equal(r, R[rows, cols]) and np.array_equal(s, S[rows, cols])


GEOMS = [
    # N, H, W, C, K, R, S, stride, pad
    (2, 8, 8, 4, 5, 3, 3, (1, 1), (1, 1)),
    (1, 9, 7, 3, 2, 3, 3, (2, 2), (1, 1)),
    (2, 6, 10, 5, 3, 3, 2, (2, 1), (0, 1)),
    (1, 7, 7, 2, 4, 1, 1, (1, 1), (0, 0)),
    (1, 5, 6, 3, 3, 3, 3, (1, 2), (2, 1)),
    (1, 10, 9, 2, 2, 4, 3, (3, 2), (1, 0)),
]


def _torch_conv_ref(x, w, dy, stride, pad):
    """float64 forward, input gradient and weight gradient from torch."""
    xt = torch.tensor(x.astype(np.float64)).permute(0, 3, 1, 2).contiguous().requires_grad_(True)
    wt = torch.tensor(w.astype(np.float64)).permute(3, 2, 0, 1).contiguous().requires_grad_(True)
    y = torch.nn.functional.conv2d(xt, wt, stride=stride, padding=pad)
    dyt = torch.tensor(dy.astype(np.float64)).permute(0, 3, 1, 2)
    y.backward(dyt)
    return (y.detach().permute(0, 2, 3, 1).numpy(),
            xt.grad.permute(0, 2, 3, 1).numpy(),
            wt.grad.permute(2, 3, 1, 0).numpy())


@pytest.mark.parametrize("geom", GEOMS)
def test_conv_exact_table_equals_torch_float64(geom):
    N, H, W, C, K, R, S, stride, pad = geom
    M = 7
    lut = oracle.lut_generate(M, "exact")
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(11, (N, H, W, C))
    w = normal(12, (R, S, C, K))
    dy = normal(13, (N, P, Q, K))
    y_ref, dx_ref, dw_ref = _torch_conv_ref(trunc(x, M), trunc(w, M), trunc(dy, M), stride, pad)
    Y, YS = oracle.conv2d_fwd(x, w, lut, M, stride, pad)
    close_to(Y, y_ref, YS)
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, lut, M, stride, pad)
    close_to(DX, dx_ref, DXS)
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, lut, M, stride, pad)
    close_to(DW, dw_ref, DWS)


def _im2col(x, R, S, stride, pad):
    """Explicit IM2COL with zero padding: rows (n, p, q), columns (r, s, c)."""
    N, H, W, C = x.shape
    sh, sw = stride
    ph, pw = pad
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    xp = np.zeros((N, H + 2 * ph + sh * 4, W + 2 * pw + sw * 4, C), np.float32)
    xp[:, ph:ph + H, pw:pw + W, :] = x
    cols = np.zeros((N, P, Q, R, S, C), np.float32)
    for r in range(R):
        for s in range(S):
            cols[:, :, :, r, s, :] = xp[:, r:r + sh * P:sh, s:s + sw * Q:sw, :]
    return cols.reshape(N * P * Q, R * S * C)


@pytest.mark.parametrize("geom", GEOMS)
def test_conv_implicit_equals_explicit_im2col_gemm(geom):
    """Same products, same order: the sums must agree bit for bit."""
    N, H, W, C, K, R, S, stride, pad = geom
    M = 7
    lut = oracle.lut_generate(M, "mitchell")
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = normal(21, (N, H, W, C))
    w = normal(22, (R, S, C, K))
    dy = normal(23, (N, P, Q, K))
    # forward: IM2COL(x) [NPQ x RSC] times W [RSC x K]
    cols = _im2col(x, R, S, stride, pad)
    Rg, Sg = oracle.gemm(cols, w.reshape(R * S * C, K), lut, M)
    Y, YS = oracle.conv2d_fwd(x, w, lut, M, stride, pad)
    assert np.array_equal(Y.reshape(-1, K), Rg) and np.array_equal(YS.reshape(-1, K), Sg)
    # weight gradient: IM2COL(x)^T [RSC x NPQ] times dY [NPQ x K]
    Rg, Sg = oracle.gemm(cols, dy.reshape(-1, K), lut, M, transA=True)
    DW, DWS = oracle.conv2d_wgrad(x, dy, w.shape, lut, M, stride, pad)
    assert np.array_equal(DW.reshape(-1, K), Rg) and np.array_equal(DWS.reshape(-1, K), Sg)
    # preceding-layer gradient: padded, dilated errors and the transposed,
    # reversed filter, then IM2COL at stride 1 and GEMM (Section VI-B)
    sh, sw = stride
    ph, pw = pad
    Hd, Wd = (P - 1) * sh + 1, (Q - 1) * sw + 1
    dil = np.zeros((N, Hd, Wd, K), np.float32)
    dil[:, ::sh, ::sw, :] = dy
    lo_h, lo_w = R - 1 - ph, S - 1 - pw
    big = np.zeros((N, H + 2 * R + Hd, W + 2 * S + Wd, K), np.float32)
    oh, ow = R + 2, S + 2   # extra margin so negative low pads stay in range
    big[:, oh + lo_h: oh + lo_h + Hd, ow + lo_w: ow + lo_w + Wd, :] = dil
    cols = np.zeros((N, H, W, R, S, K), np.float32)
    for r in range(R):
        for s in range(S):
            # row h of dx reads padded-dilated row h + (R-1-r), i.e. filter row r
            cols[:, :, :, r, s, :] = big[:, oh + R - 1 - r: oh + R - 1 - r + H, ow + S - 1 - s: ow + S - 1 - s + W, :]
    wt = w.transpose(0, 1, 3, 2).reshape(R * S * K, C)   # transposed (C <-> K), rows (r, s, k)
    Rg, Sg = oracle.gemm(cols.reshape(N * H * W, R * S * K), wt, lut, M)
    DX, DXS = oracle.conv2d_dgrad(dy, w, x.shape, lut, M, stride, pad)
    assert np.array_equal(DX.reshape(-1, C), Rg) and np.array_equal(DXS.reshape(-1, C), Sg)


def test_conv_sampled_outputs_match_full_pass():
    geom = GEOMS[1]
    N, H, W, C, K, R, S, stride, pad = geom
    lut = oracle.lut_generate(7, "mitchell")
    P, Q = oracle.conv_out_hw(H, W, R, S, stride, pad)
    x = uniform(31, (N, H, W, C))
    w = normal(32, (R, S, C, K))
    dy = normal(33, (N, P, Q, K))
    for fn, args, shape in (
        (oracle.conv2d_fwd, (x, w), (N, P, Q, K)),
        (oracle.conv2d_dgrad, (dy, w, x.shape), (N, H, W, C)),
        (oracle.conv2d_wgrad, (x, dy, w.shape), (R, S, C, K)),
    ):
        full, fulls = fn(*args, lut, 7, stride, pad)
        idx = np.array([0, 3, int(np.prod(shape)) - 1, 7])
        r, s = fn(*args, lut, 7, stride, pad, idx=idx)
        assert np.array_equal(r, full.ravel()[idx]) and np.array_equal(s, fulls.ravel()[idx])


def test_conv_padding_is_a_multiplied_zero():
    """Padding slots are zero operands (the IM2COL buffer holds zeros), so an
    infinite weight facing padding gives NaN (0 * Inf), as it would through
    IM2COL + GEMM."""
    lut = oracle.lut_generate(7, "exact")
    x = np.ones((1, 4, 4, 1), np.float32)
    w = np.ones((3, 3, 1, 1), np.float32)
    w[0, 0, 0, 0] = np.inf
    Y, _ = oracle.conv2d_fwd(x, w, lut, 7, (1, 1), (1, 1))
    assert np.isnan(Y[0, 0, 0, 0]) and np.isnan(Y[0, 0, 3, 0])   # top row faces padding at r=0
    assert np.isinf(Y[0, 1, 1, 0]) and Y[0, 1, 1, 0] > 0          # interior sees x=1 there
