"""Comparison of GPU results with the oracle.

Gate (the reading of "max relative error 1e-5" that FP32 accumulation can
meet): for every output, |c - r| <= tol * S, where r is the oracle's float64
sum of the same approximate products and S the float64 sum of their
magnitudes; S = 0 requires c = 0. Non-finite oracle values must be matched
exactly (same infinity, or NaN for NaN).
"""
import numpy as np

TOL = 1e-5


def gate(c, r, s, tol=TOL, what=""):
    c = np.asarray(c, dtype=np.float64).ravel()
    r = np.asarray(r, dtype=np.float64).ravel()
    s = np.asarray(s, dtype=np.float64).ravel()
    assert c.shape == r.shape == s.shape, (c.shape, r.shape, s.shape)
    fin = np.isfinite(r) & np.isfinite(s)
    nan_r = np.isnan(r) | (np.isnan(s) & ~np.isinf(r))
    if np.any(nan_r):
        assert np.all(np.isnan(c[nan_r])), f"{what}: expected NaN"
    inf_r = np.isinf(r) & ~nan_r
    if np.any(inf_r):
        assert np.array_equal(c[inf_r], r[inf_r]), f"{what}: expected matching infinities"
    # finite oracle sums whose magnitudes overflow double would be a test bug
    cf, rf, sf = c[fin], r[fin], s[fin]
    assert np.all(np.isfinite(cf)), f"{what}: non-finite result where the oracle is finite"
    zero = sf == 0
    assert np.all(cf[zero] == 0), f"{what}: non-zero result where every product is zero"
    err = np.abs(cf[~zero] - rf[~zero]) / sf[~zero]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{what}: max |c-r|/S = {worst:.3e} > {tol}"
    return worst


def same_bits(c, want, what="", zero_sign=True):
    """Bitwise equality of float32 results with the oracle's FP32-order sums
    (reading R20): NaN matches any NaN; with zero_sign False, +0 and -0 match
    each other (the native multiplier leaves the sign of a zero sum open)."""
    c = np.ascontiguousarray(c, dtype=np.float32).ravel()
    w = np.ascontiguousarray(want, dtype=np.float32).ravel()
    assert c.shape == w.shape, (c.shape, w.shape)
    cn, wn = np.isnan(c), np.isnan(w)
    assert np.array_equal(cn, wn), f"{what}: NaN at {np.flatnonzero(cn != wn)[:8]}"
    cb, wb = c.view(np.uint32), w.view(np.uint32)
    diff = (cb != wb) & ~cn
    if not zero_sign:
        diff &= ~((c == 0) & (w == 0))
    bad = np.flatnonzero(diff)
    assert bad.size == 0, (f"{what}: {bad.size} of {c.size} outputs differ from the FP32-order sums, "
                           f"first at {bad[:4]}: got {c[bad[:4]]}, want {w[bad[:4]]}")
    return c.size
