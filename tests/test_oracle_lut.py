"""Pins of the oracle's table generation (Algorithm 1 of "ApproxTrain",
arXiv 2209.04161, Section V-A) against closed forms and hand-worked values."""
import os

import numpy as np
import pytest

import oracle
from datagen import PERTURB_SEED, pm_one

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def exact_entries_closed_form(M):
    """Integer closed form of the exact mantissa product: P = (2^M+ia)(2^M+ib)
    over 2^(2M); carry when P >= 2^(2M+1); the 15-bit fraction is truncated."""
    ia, ib = np.meshgrid(np.arange(1 << M), np.arange(1 << M), indexing="ij")
    P = ((1 << M) + ia.astype(np.int64)) * ((1 << M) + ib.astype(np.int64))
    carry = (P >= (1 << (2 * M + 1))).astype(np.int64)
    base = np.int64(1) << (2 * M + carry)           # 2^(2M) or 2^(2M+1)
    frac15 = ((P - base) << 15) // base             # floor of the fraction * 2^15
    return ((carry << 15) | frac15).astype(np.uint16).ravel()


def mitchell_entries_closed_form(M):
    """Mitchell: x = ia/2^M, y = ib/2^M. Value 1+x+y (carry 0) when ia+ib < 2^M,
    else 2(x+y) = 2(1 + (x+y-1)) (carry 1, fraction x+y-1)."""
    ia, ib = np.meshgrid(np.arange(1 << M), np.arange(1 << M), indexing="ij")
    s = ia.astype(np.int64) + ib
    carry = (s >= (1 << M)).astype(np.int64)
    frac15 = (s - (carry << M)) << (15 - M)
    return ((carry << 15) | frac15).astype(np.uint16).ravel()


# M = 9..11: the tables the library reads from global memory (Section V gives
# m up to 11). The model's FP32 product of two (M+1)-bit significands is exact
# up to M = 11 (24 bits), so the closed forms hold over the whole range.
@pytest.mark.parametrize("M", list(range(1, 12)))
def test_exact_table_matches_integer_closed_form(M):
    assert np.array_equal(oracle.lut_generate(M, "exact"), exact_entries_closed_form(M))


@pytest.mark.parametrize("M", list(range(1, 12)))
def test_mitchell_table_matches_integer_closed_form(M):
    assert np.array_equal(oracle.lut_generate(M, "mitchell"), mitchell_entries_closed_form(M))


def test_exact_table_needs_no_truncation_up_to_m7_but_does_at_m8():
    # (M+1)-bit significands give a 2M+2 bit product: fraction <= 2M+1 <= 15 bits for M <= 7
    for M in range(1, 8):
        ia, ib = np.meshgrid(np.arange(1 << M), np.arange(1 << M), indexing="ij")
        P = ((1 << M) + ia.astype(np.int64)) * ((1 << M) + ib.astype(np.int64))
        lut = oracle.lut_generate(M, "exact").astype(np.int64).reshape(P.shape)
        carry, f = lut >> 15, lut & 0x7FFF
        value = (1.0 + f / 32768.0) * (1 << carry) * (1 << (2 * M))
        assert np.array_equal(value, P.astype(np.float64))
    # at M = 8 the 17-bit fraction is chopped to 15 bits: never rounded up,
    # and off by less than one unit of the 15-bit field
    M = 8
    lut8 = oracle.lut_generate(M, "exact").astype(np.int64).reshape(256, 256)
    ia, ib = np.meshgrid(np.arange(256), np.arange(256), indexing="ij")
    P = ((256 + ia.astype(np.int64)) * (256 + ib.astype(np.int64))).astype(np.float64)
    carry, f = lut8 >> 15, lut8 & 0x7FFF
    value = (1.0 + f / 32768.0) * (1 << carry) * (1 << (2 * M))
    err = P - value
    assert np.all(err >= 0)
    assert np.all(err < (1 << carry) * (1 << (2 * M)) / 32768.0)
    assert np.count_nonzero(err) > 0


def test_hand_entries():
    lut = oracle.lut_generate(7, "exact")
    assert lut[(64 << 7) | 64] == 0x9000      # 1.5 * 1.5 = 2 * 1.125
    assert lut[(32 << 7) | 32] == 0x4800      # 1.25 * 1.25 = 1.5625
    assert lut[0] == 0x0000                   # 1 * 1
    mit = oracle.lut_generate(7, "mitchell")
    assert mit[(64 << 7) | 64] == 0x8000      # x+y = 1 -> 2.0
    assert mit[(32 << 7) | 32] == 0x4000      # 1.5


def test_generic_model_callback_gives_the_same_table():
    # Algorithm 1 only sees the model through its outputs
    for M in (3, 5):
        via_cb = oracle.lut_generate(M, lambda a, b: np.float32(a) * np.float32(b))
        assert np.array_equal(via_cb, oracle.lut_generate(M, "exact"))


def test_algorithm1_rejects_products_below_one():
    with pytest.raises(ValueError):
        oracle.lut_generate(4, lambda a, b: 0.25 * a * b)


def test_perturbed_table():
    M = 8
    base = oracle.lut_generate(M, "exact")
    delta = pm_one(PERTURB_SEED, 1 << 16)
    pert = oracle.lut_perturb(M, base, delta)
    b = base.astype(np.int64)
    p = pert.astype(np.int64)
    assert np.array_equal(b >> 15, p >> 15)              # carry untouched
    d = (p & 0x7FFF) - (b & 0x7FFF)
    sat = ((b & 0x7FFF) == 0) & (delta < 0) | ((b & 0x7FFF) == 0x7FFF) & (delta > 0)
    assert np.array_equal(d[~sat], delta[~sat].astype(np.int64))
    assert np.all(d[sat] == 0)
    assert 0.45 < np.mean(delta > 0) < 0.55
    # the table is no longer symmetric: operand order matters
    t = p.reshape(256, 256)
    assert np.count_nonzero(t != t.T) > 1000


def test_datagen_generator_matches_published_splitmix64():
    """First outputs of splitmix64 seeded with 1234567, as printed by the
    reference implementation of the generator (Steele, Lea and Flood 2014)."""
    from datagen import splitmix64
    assert [int(v) for v in splitmix64(1234567, 3)] == [
        6457827717110365317, 3203168211198807973, 9817491932198370423]
