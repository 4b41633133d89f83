"""Pins of the oracle's product rule (Algorithm 2 of "ApproxTrain",
arXiv 2209.04161, Section V): hand-worked values, IEEE equivalence with the
exact table, exhaustive brute force at small M, and invariants."""
import os

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, normal, pm_one, special_values, splitmix64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lut(model, M):
    if model == "perturbed":
        return oracle.lut_perturb(M, oracle.lut_generate(M, "exact"), pm_one(PERTURB_SEED, 1 << (2 * M)))
    return oracle.lut_generate(M, model)


def test_golden_products():
    rows = []
    with open(os.path.join(GOLDEN, "hand_products.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                model, M, a, b, want = line.split()
                rows.append((model, int(M), int(a, 16), int(b, 16), int(want, 16)))
    assert len(rows) >= 20
    for model, M, a, b, want in rows:
        got = int(oracle.amsim_bits(np.array([a], np.uint32), np.array([b], np.uint32), _lut(model, M), M)[0])
        assert got == want, (model, hex(a), hex(b), hex(got), hex(want))


def _daz_trunc(bits, M):
    """DAZ (subnormal -> signed zero) then keep the top M fraction bits."""
    bits = bits.astype(np.uint32)
    e = (bits >> 23) & 0xFF
    out = np.where(e == 0, bits & 0x80000000, bits & np.uint32(~((1 << (23 - M)) - 1) & 0xFFFFFFFF))
    # keep NaN payloads NaN after chopping (a NaN with only low payload bits would become Inf)
    nan = (e == 255) & ((bits & 0x7FFFFF) != 0)
    return np.where(nan, np.uint32(0x7FC00000), out).astype(np.uint32)


def _ftz(x):
    x = x.astype(np.float32)
    tiny = np.abs(x) < np.float32(2.0 ** -126)
    return np.where(tiny & (x != 0), np.copysign(np.float32(0), x), x).astype(np.float32)


def _random_bits(seed, n):
    return (splitmix64(seed, n) >> np.uint64(32)).astype(np.uint32)


@pytest.mark.parametrize("M", [1, 2, 3, 5, 7])
def test_exact_table_equals_ieee_product_of_truncated_operands(M):
    """With the exact table, the rule is FTZ(fp32(trunc(DAZ a) * trunc(DAZ b)))
    for every input: the product of two (M+1)-bit significands is exact in
    FP32, and IEEE overflow gives infinity where the rule does."""
    lut = _lut("exact", M)
    n = 400_000
    a = _random_bits(11 + M, n)
    b = _random_bits(23 + M, n)
    # add normals of moderate size and every pair of special values
    nm = normal(5 + M, (20000,)).view(np.uint32)
    sp = special_values().view(np.uint32)
    spa, spb = np.meshgrid(sp, sp, indexing="ij")
    a = np.concatenate([a, nm, np.roll(nm, 7), spa.ravel(), sp, nm[: sp.size]])
    b = np.concatenate([b, np.roll(nm, 3), nm, spb.ravel(), nm[: sp.size], sp])
    got = oracle.amsim_bits(a, b, lut, M)
    with np.errstate(all="ignore"):
        ref = _ftz(_daz_trunc(a, M).view(np.float32) * _daz_trunc(b, M).view(np.float32)).view(np.uint32)
    gnan = np.isnan(got.view(np.float32))
    rnan = np.isnan(ref.view(np.float32))
    assert np.array_equal(gnan, rnan)
    assert np.array_equal(got[~gnan], ref[~rnan])
    assert np.all(got[gnan] == 0x7FC00000)


@pytest.mark.parametrize("model", ["exact", "mitchell"])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_brute_force_every_mantissa_exponent_sign_combination(model, M):
    """All 2^M x 2^M mantissa pairs x all 254 x 254 normal exponent pairs x 4
    sign pairs, against the mathematical value of the model's product,
    flushed to zero below 2^-126 and saturated to infinity from 2^128."""
    lut = _lut(model, M)
    nm = 1 << M
    ia, ib = np.meshgrid(np.arange(nm, dtype=np.int64), np.arange(nm, dtype=np.int64), indexing="ij")
    ia, ib = ia.ravel(), ib.ravel()
    x, y = ia / nm, ib / nm
    if model == "exact":
        sig = (1.0 + x) * (1.0 + y)
    else:
        sig = np.where(x + y < 1.0, 1.0 + x + y, 2.0 * (x + y))
    eb = np.arange(1, 255, dtype=np.int64)
    for sa in (0, 1):
        for sb in (0, 1):
            for ea in range(1, 255):
                A = ((sa << 31) | (ea << 23) | (ia << (23 - M)))[:, None] + 0 * eb[None, :]
                B = ((sb << 31) | (eb[None, :] << 23) | (ib << (23 - M))[:, None])
                got = oracle.amsim_bits(A.astype(np.uint32), B.astype(np.uint32), lut, M).view(np.float32)
                v = sig[:, None] * np.exp2((ea + eb[None, :] - 254).astype(np.float64))
                v = np.where(v < 2.0 ** -126, 0.0, v)
                v = np.where(v >= 2.0 ** 128, np.inf, v)
                if sa ^ sb:
                    v = -v
                assert np.array_equal(got.astype(np.float64), v), (model, M, sa, sb, ea)
                # zero results carry the XOR sign
                z = v == 0
                assert np.all(np.signbit(got[z]) == bool(sa ^ sb))


@pytest.mark.parametrize("model", ["exact", "mitchell", "perturbed"])
def test_invariants(model):
    M = 8 if model == "perturbed" else 7
    lut = _lut(model, M)
    a = normal(101, (50000,))
    b = normal(102, (50000,))
    p = oracle.amsim(a, b, lut, M)
    # sign symmetry
    assert np.array_equal(oracle.amsim(-a, b, lut, M), -p)
    assert np.array_equal(oracle.amsim(a, -b, lut, M), -p)
    assert np.array_equal(oracle.amsim(-a, -b, lut, M), p)
    # zero operands give signed zeros
    z = oracle.amsim(np.zeros_like(a), b, lut, M)
    assert np.all(z == 0) and np.array_equal(np.signbit(z), np.signbit(b))
    # power-of-two scaling of either operand scales the product (no under/overflow here)
    for j in (-40, -3, 1, 17, 60):
        s = np.float32(2.0 ** j)
        assert np.array_equal(oracle.amsim(a * s, b, lut, M), p * s)
        assert np.array_equal(oracle.amsim(a, b * s, lut, M), p * s)
    # the product sees an operand only through sign, exponent and top M fraction bits
    low = (splitmix64(103, a.size) & np.uint64((1 << (23 - M)) - 1)).astype(np.uint32)
    a2 = (a.view(np.uint32) ^ low).view(np.float32)
    b2 = (b.view(np.uint32) ^ np.roll(low, 5)).view(np.float32)
    assert np.array_equal(oracle.amsim(a2, b2, lut, M), p)
    # every product's low 8 mantissa bits are zero (15-bit table mantissa)
    assert np.all((p.view(np.uint32) & 0xFF) == 0)
    q = oracle.amsim(b, a, lut, M)
    if model == "perturbed":
        assert np.count_nonzero(q != p) > 100      # operand order is exercised
    else:
        assert np.array_equal(q, p)                # symmetric tables commute


def test_mitchell_never_overestimates_and_is_within_one_ninth():
    """Mitchell's product of the truncated operands lies in [8/9, 1] times the
    exact product of the same truncated operands (worst case x = y = 1/2)."""
    M = 7
    a = normal(201, (200000,))
    b = normal(202, (200000,))
    mit = oracle.amsim(a, b, _lut("mitchell", M), M).astype(np.float64)
    ex = oracle.amsim(a, b, _lut("exact", M), M).astype(np.float64)
    r = mit / ex
    assert np.all(r <= 1.0) and np.all(r >= 8.0 / 9.0 - 1e-12)
    assert r.min() < 0.9  # the bound is approached


def test_index_order_first_operand_in_high_bits():
    """The index concatenates the first operand's mantissa above the
    second's: with entry[i] = i (carry 0) the product's fraction field shows
    (ia << M | ib) << 8."""
    M = 4
    lut = np.arange(1 << (2 * M), dtype=np.uint16)
    ia, ib = np.meshgrid(np.arange(16, dtype=np.uint32), np.arange(16, dtype=np.uint32), indexing="ij")
    A = (127 << 23) | (ia.ravel() << 19)
    B = (127 << 23) | (ib.ravel() << 19)
    got = oracle.amsim_bits(A.astype(np.uint32), B.astype(np.uint32), lut, M)
    assert np.array_equal(got & 0x7FFFFF, ((ia.ravel() << M) | ib.ravel()) << 8)
    assert np.all((got >> 23) == 127)
