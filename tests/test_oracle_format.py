"""Pins of the oracle's (1, E, M) formats: the exponent cast and the
format's range in Algorithm 2 ("ApproxTrain", arXiv 2209.04161, Section V:
exponent widths 1 to 8 given an exponent cast). Hand-worked values, and with
the exact table a closed form computed here from the definition of the
format (independent of the oracle's code), over random operands and
exhaustively at small M."""
import math
import os

import numpy as np
import pytest

import oracle
from datagen import splitmix64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_format_products():
    rows = []
    with open(os.path.join(GOLDEN, "format_products.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                model, M, E, a, b, want = line.split()
                rows.append((model, int(M), int(E), int(a, 16), int(b, 16), int(want, 16)))
    assert len(rows) >= 25
    for model, M, E, a, b, want in rows:
        lut = oracle.lut_generate(M, model)
        got = int(oracle.amsim_bits(np.array([a], np.uint32), np.array([b], np.uint32), lut, M, E)[0])
        assert got == want, (model, M, E, hex(a), hex(b), hex(got), hex(want))


def _expected_exact(a, b, M, E):
    """The exact multiplier in (1, E, M), from the definition: cast each
    operand to E exponent bits (bias 2^(E-1)-1, normal unbiased exponents
    1-bias..bias, no subnormals), chop it to M fraction bits, multiply exactly,
    and cast the product the same way. Returns the float value (NaN, +-Inf,
    +-0 included)."""
    bias = (1 << (E - 1)) - 1

    def cast(x):
        if math.isnan(x) or math.isinf(x) or x == 0.0:
            return x
        m, ex = math.frexp(abs(x))          # abs(x) = m 2^ex, m in [0.5, 1)
        u = ex - 1                          # unbiased exponent of 1.f form
        if u < -126:                        # FP32 subnormal input: zero
            return math.copysign(0.0, x)
        if u < 1 - bias:
            return math.copysign(0.0, x)
        if u > bias:
            return math.copysign(math.inf, x)
        sig = math.floor(m * 2 * (1 << M)) / (1 << M)       # 1.f chopped to M bits
        return math.copysign(math.ldexp(sig, u), x)

    ca, cb = cast(a), cast(b)
    sign = -1.0 if (math.copysign(1.0, a) * math.copysign(1.0, b)) < 0 else 1.0
    if math.isnan(ca) or math.isnan(cb):
        return math.nan
    if math.isinf(ca) or math.isinf(cb):
        if ca == 0.0 or cb == 0.0:
            return math.nan
        return sign * math.inf
    if ca == 0.0 or cb == 0.0:
        return sign * 0.0
    p = abs(ca) * abs(cb)                   # exact in double (<= 2 x 8 significant bits)
    u = math.frexp(p)[1] - 1
    if u < 1 - bias:
        return sign * 0.0
    if u > bias:
        return sign * math.inf
    return sign * p


def _check(a_bits, b_bits, M, E, lut):
    got = oracle.amsim_bits(a_bits, b_bits, lut, M, E).view(np.float32)
    for x, y, g in zip(a_bits.view(np.float32), b_bits.view(np.float32), got):
        w = _expected_exact(float(x), float(y), M, E)
        if math.isnan(w):
            assert np.isnan(g), (x, y, E)
        else:
            assert float(g) == w and math.copysign(1.0, float(g)) == math.copysign(1.0, w), (x, y, M, E, g, w)


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("M", [3, 7])
def test_exact_table_is_the_cast_chopped_product(M, E):
    lut = oracle.lut_generate(M, "exact")
    bias = (1 << (E - 1)) - 1
    n = 3000
    r = splitmix64(7000 + 10 * E + M, 3 * n)
    sign = (r[0::3] & np.uint64(1)).astype(np.uint32) << np.uint32(31)
    # exponents from a little below to a little above the format's range
    lo, hi = max(1, 127 - bias - 3), min(254, 127 + bias + 3)
    exp = (lo + (r[1::3] % np.uint64(hi - lo + 1))).astype(np.uint32)
    frac = (r[2::3] >> np.uint64(41)).astype(np.uint32) & np.uint32(0x7FFFFF)
    bits = sign | (exp << np.uint32(23)) | frac
    sp = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x00400000], np.uint32)
    a = np.concatenate([bits[: n // 2], np.repeat(sp, 6)])
    b = np.concatenate([bits[n // 2: n // 2 * 2], np.tile(sp, 6)])
    _check(a, b, M, E, lut)


@pytest.mark.parametrize("E", [2, 3, 4])
def test_brute_force_small_formats(E):
    """M = 2: every mantissa pair, every exponent pair from 2 below to 2 above
    the format's range, both signs."""
    M = 2
    lut = oracle.lut_generate(M, "exact")
    bias = (1 << (E - 1)) - 1
    exps = np.arange(127 - bias - 2, 127 + bias + 3, dtype=np.uint32)
    vals = [(s << 31) | (e << 23) | (m << 21) for s in (0, 1) for e in exps for m in range(4)]
    vals = np.array(vals, dtype=np.uint32)
    a = np.repeat(vals, vals.size)
    b = np.tile(vals, vals.size)
    _check(a, b, M, E, lut)


def test_cast_is_identity_at_fp32_range():
    r = splitmix64(77, 4000).astype(np.uint32)
    assert np.array_equal(oracle.cast_bits(r, 8), r)


def test_gemm_in_range_equals_float64_matmul_of_chopped_operands():
    """E = 5 with every operand and product inside the format's range: the
    exact-table GEMM is the float64 product of the M-bit-chopped matrices."""
    M, E = 7, 5
    lut = oracle.lut_generate(M, "exact")
    rng = np.random.default_rng(5)
    A = (rng.uniform(1, 2, (9, 11)) * 2.0 ** rng.integers(-6, 6, (9, 11))).astype(np.float32)
    B = (rng.uniform(1, 2, (11, 7)) * 2.0 ** rng.integers(-6, 6, (11, 7))).astype(np.float32)
    A *= np.where(rng.random(A.shape) < 0.5, -1, 1).astype(np.float32)
    chop = lambda X: (X.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    R, S = oracle.gemm(A, B, lut, M, E=E)
    assert np.array_equal(R, chop(A) @ chop(B))
    assert np.array_equal(S, np.abs(chop(A)) @ np.abs(chop(B)))


def test_gemm_products_under_and_over_the_range():
    """Products below the E = 4 range vanish from the sum, inputs above it
    make it infinite."""
    M, E = 7, 4                      # bias 7: normal 2^-6 .. 2^7
    lut = oracle.lut_generate(M, "exact")
    A = np.array([[2.0 ** -4, 1.0, 2.0 ** -3]], np.float32)        # 1 x 3
    B = np.array([[2.0 ** -3], [1.5], [2.0 ** -2]], np.float32)    # 3 x 1
    R, S = oracle.gemm(A, B, lut, M, E=E)
    # 2^-7 (below 2^-6) -> 0; 1.5; 2^-5 -> kept
    assert R[0, 0] == 1.5 + 2.0 ** -5 and S[0, 0] == 1.5 + 2.0 ** -5
    A2 = np.array([[256.0, 1.0]], np.float32)                     # 2^8 casts to Inf
    B2 = np.array([[1.0], [1.0]], np.float32)
    R2, _ = oracle.gemm(A2, B2, lut, M, E=E)
    assert np.isinf(R2[0, 0]) and R2[0, 0] > 0
