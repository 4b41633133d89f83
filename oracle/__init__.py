"""Oracle: plain CPU reference of LUT-based approximate FP32 multiplication.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product library does not import
it, and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C99, single-threaded, double
accumulation); this module only builds and loads it and marshals numpy arrays.
Sources: "ApproxTrain: Fast Simulation of Approximate Multipliers for DNN
Training and Inference" (arXiv 2209.04161) -- Section V-A Algorithm 1 (table
generation), Section V Algorithm 2 (AMSim product; the (1, e, m) formats with
an exponent cast), Section VI-B Algorithms 3-4 (Conv2D forward and backprop).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MUL_FN = ctypes.CFUNCTYPE(ctypes.c_float, ctypes.c_float, ctypes.c_float)


def build():
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-o", _LIB, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        c_int, c_i64 = ctypes.c_int, ctypes.c_int64
        vp = ctypes.c_void_p
        L.orc_mul_exact.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_mul_exact.restype = ctypes.c_float
        L.orc_mul_mitchell.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_mul_mitchell.restype = ctypes.c_float
        L.orc_mul_native.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_mul_native.restype = ctypes.c_double
        L.orc_lut_generate.argtypes = [c_int, vp, vp]
        L.orc_lut_generate.restype = c_int
        L.orc_lut_perturb.argtypes = [c_int, vp, vp]
        L.orc_lut_perturb.restype = None
        L.orc_amsim_bits.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp, c_int]
        L.orc_amsim_bits.restype = ctypes.c_uint32
        L.orc_amsim_bits_fmt.argtypes = [ctypes.c_uint32, ctypes.c_uint32, vp, c_int, c_int]
        L.orc_amsim_bits_fmt.restype = ctypes.c_uint32
        L.orc_cast_bits.argtypes = [ctypes.c_uint32, c_int]
        L.orc_cast_bits.restype = ctypes.c_uint32
        L.orc_amsim_many.argtypes = [c_i64, vp, vp, vp, c_int, c_int, vp]
        L.orc_amsim_many.restype = None
        L.orc_gemm.argtypes = [c_int] * 5 + [vp, c_int, vp, c_int, vp, c_int, c_int, vp, vp]
        L.orc_gemm.restype = None
        L.orc_gemm_at.argtypes = [c_int] * 5 + [vp, c_int, vp, c_int, vp, c_int, c_int,
                                                 c_i64, vp, vp, vp, vp]
        L.orc_gemm_at.restype = None
        L.orc_gemm_f32_at.argtypes = [c_int] * 5 + [vp, c_int, vp, c_int, vp, c_int, c_int,
                                                     c_i64, vp, vp, vp, vp]
        L.orc_gemm_f32_at.restype = None
        L.orc_conv2d_f32.argtypes = [c_int] * 12 + [vp, vp, vp, c_int, c_int, c_i64, vp, vp, vp]
        L.orc_conv2d_f32.restype = None
        for name in ("orc_conv2d_fwd", "orc_conv2d_dgrad", "orc_conv2d_wgrad"):
            f = getattr(L, name)
            f.argtypes = [c_int] * 11 + [vp, vp, vp, c_int, c_int, c_i64, vp, vp, vp]
            f.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _table(lut, M):
    """(table array or None, pointer, M) for the C calls. lut=None selects
    the native multiplier (exact products; M must then be 0)."""
    if lut is None:
        assert M == 0
        return None, None, 0
    t = np.ascontiguousarray(lut, dtype=np.uint16)
    return t, _ptr(t), M


# ---------------------------------------------------------------- tables

def lut_generate(M, model):
    """Algorithm 1. ``model`` is "exact", "mitchell" or a Python callable
    float(float, float). Returns a uint16 array of 4**M entries."""
    L = lib()
    out = np.zeros(1 << (2 * M), dtype=np.uint16)
    keep = None
    if model == "exact":
        fp = ctypes.cast(L.orc_mul_exact, ctypes.c_void_p)
    elif model == "mitchell":
        fp = ctypes.cast(L.orc_mul_mitchell, ctypes.c_void_p)
    else:
        keep = MUL_FN(lambda a, b: float(model(a, b)))
        fp = ctypes.cast(keep, ctypes.c_void_p)
    rc = L.orc_lut_generate(M, fp, _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_lut_generate failed with {rc}")
    return out


def lut_perturb(M, lut, delta):
    """Move each entry's mantissa field by delta (+1/-1), saturating; carry kept."""
    out = np.array(lut, dtype=np.uint16, copy=True)
    d = np.ascontiguousarray(delta, dtype=np.int8)
    assert d.size == out.size == (1 << (2 * M))
    lib().orc_lut_perturb(M, _ptr(out), _ptr(d))
    return out


# ---------------------------------------------------------------- products

def amsim_bits(a_bits, b_bits, lut, M, E=8):
    """Algorithm 2 element-wise on uint32 bit patterns (same shapes), in the
    format (1, E, M): operands cast to E exponent bits first (E = 8: FP32)."""
    a = np.ascontiguousarray(a_bits, dtype=np.uint32).ravel()
    b = np.ascontiguousarray(b_bits, dtype=np.uint32).ravel()
    assert a.size == b.size
    lut = np.ascontiguousarray(lut, dtype=np.uint16)
    out = np.empty_like(a)
    lib().orc_amsim_many(a.size, _ptr(a), _ptr(b), _ptr(lut), M, E, _ptr(out))
    return out.reshape(np.shape(a_bits))


def amsim(a, b, lut, M, E=8):
    """Algorithm 2 on float32 arrays; returns float32."""
    a = _f32(a)
    b = _f32(b)
    return amsim_bits(a.view(np.uint32), b.view(np.uint32), lut, M, E).view(np.float32)


def cast_bits(x_bits, E):
    """The exponent cast of FP32 bit patterns to E exponent bits."""
    f = lib().orc_cast_bits
    x = np.ascontiguousarray(x_bits, dtype=np.uint32).ravel()
    return np.array([f(int(v), E) for v in x], dtype=np.uint32).reshape(np.shape(x_bits))


def mul_native(a, b):
    """The native multiplier (exact product of two floats, as float64)."""
    a = _f32(a).ravel()
    b = _f32(b).ravel()
    f = lib().orc_mul_native
    return np.array([f(float(x), float(y)) for x, y in zip(a, b)], dtype=np.float64)


# ---------------------------------------------------------------- GEMM

def gemm(A, B, lut, M, transA=False, transB=False, E=8):
    """R = sum of approximate products (float64) and S = sum of their
    magnitudes, for op(A) @ op(B). A and B are 2-D float32 arrays stored
    row-major (op = transpose of the stored matrix when trans is set).
    E: exponent bits of the multiplier's format (8 = FP32)."""
    A = _f32(A)
    B = _f32(B)
    m = A.shape[1] if transA else A.shape[0]
    k = A.shape[0] if transA else A.shape[1]
    kb = B.shape[1] if transB else B.shape[0]
    n = B.shape[0] if transB else B.shape[1]
    assert k == kb
    R = np.zeros((m, n), dtype=np.float64)
    S = np.zeros((m, n), dtype=np.float64)
    t, tp, M = _table(lut, M)
    lib().orc_gemm(int(transA), int(transB), m, n, k, _ptr(A), A.shape[1],
                   _ptr(B), B.shape[1], tp, M, E, _ptr(R), _ptr(S))
    return R, S


def default_threads():
    """Host threads for the threaded driver: the cores this process may use,
    at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _threaded(count, threads, run):
    """The threaded driver: run(lo, hi) computes outputs [lo, hi) with the
    same per-output C code and returns a tuple of arrays; the output range is
    cut into `threads` disjoint blocks run side by side (ctypes releases the
    interpreter lock during the C calls). threads None or 1: one call."""
    if not threads or threads <= 1 or count < 2 * threads:
        return run(0, count)
    from concurrent.futures import ThreadPoolExecutor
    bounds = np.linspace(0, count, threads + 1).astype(np.int64)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda i: run(int(bounds[i]), int(bounds[i + 1])), range(threads)))
    return tuple(np.concatenate([p[j] for p in parts]) for j in range(len(parts[0])))


def gemm_at(A, B, lut, M, rows, cols, transA=False, transB=False, E=8, threads=None):
    """The same sums at the (rows[t], cols[t]) outputs only (threads: the
    threaded driver over disjoint blocks of the outputs)."""
    A = _f32(A)
    B = _f32(B)
    m = A.shape[1] if transA else A.shape[0]
    k = A.shape[0] if transA else A.shape[1]
    n = B.shape[0] if transB else B.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int32).ravel()
    cols = np.ascontiguousarray(cols, dtype=np.int32).ravel()
    assert rows.shape == cols.shape
    t, tp, M = _table(lut, M)

    def run(lo, hi):
        R = np.zeros(hi - lo, dtype=np.float64)
        S = np.zeros(hi - lo, dtype=np.float64)
        r, c = rows[lo:hi], cols[lo:hi]
        lib().orc_gemm_at(int(transA), int(transB), m, n, k, _ptr(A), A.shape[1],
                          _ptr(B), B.shape[1], tp, M, E, hi - lo,
                          _ptr(r), _ptr(c), _ptr(R), _ptr(S))
        return R, S

    return _threaded(rows.size, threads, run)


def _chunks(chunk, count):
    c = np.ascontiguousarray(np.broadcast_to(np.asarray(chunk, dtype=np.int64), (count,)))
    assert np.all(c > 0)
    return c


def gemm_f32_at(A, B, lut, M, rows, cols, chunk, transA=False, transB=False, E=8, threads=None):
    """The FP32 sums in the documented order (reading R20) at the outputs
    (rows[t], cols[t]): reduction chunks of chunk[t] indices (a scalar
    applies to every output; chunk >= k means one chunk). float32 array."""
    A = _f32(A)
    B = _f32(B)
    m = A.shape[1] if transA else A.shape[0]
    k = A.shape[0] if transA else A.shape[1]
    n = B.shape[0] if transB else B.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int32).ravel()
    cols = np.ascontiguousarray(cols, dtype=np.int32).ravel()
    assert rows.shape == cols.shape
    ch = _chunks(chunk, rows.size)
    t, tp, M = _table(lut, M)

    def run(lo, hi):
        out = np.zeros(hi - lo, dtype=np.float32)
        r, c, cc = rows[lo:hi], cols[lo:hi], ch[lo:hi]
        lib().orc_gemm_f32_at(int(transA), int(transB), m, n, k, _ptr(A), A.shape[1],
                              _ptr(B), B.shape[1], tp, M, E, hi - lo,
                              _ptr(r), _ptr(c), _ptr(cc), _ptr(out))
        return (out,)

    return _threaded(rows.size, threads, run)[0]


def gemm_f32(A, B, lut, M, chunk, transA=False, transB=False, E=8):
    """gemm_f32_at over every output; chunk: scalar or an m x n array."""
    m = A.shape[1] if transA else A.shape[0]
    n = B.shape[0] if transB else B.shape[1]
    rows, cols = np.meshgrid(np.arange(m, dtype=np.int32), np.arange(n, dtype=np.int32), indexing="ij")
    ch = np.broadcast_to(np.asarray(chunk, dtype=np.int64), (m, n)).ravel()
    return gemm_f32_at(A, B, lut, M, rows.ravel(), cols.ravel(), ch, transA, transB, E).reshape(m, n)


CONV_PASSES = {"fwd": 0, "dgrad": 1, "wgrad": 2}


def conv2d_f32(pass_name, t1, t2, geom, lut, M, chunk, idx=None, E=8, threads=None):
    """FP32 sums of a Conv2D pass in the documented order (reading R20) at
    flat output indices idx (all outputs when None). geom = (N, H, W, C, K,
    R, S, (sh, sw), (ph, pw)); t1, t2 as for conv2d_fwd / dgrad / wgrad
    (x, w / dy, w / x, dy)."""
    N, H, W, C, K, R, S, (sh, sw), (ph, pw) = geom
    P, Q = conv_out_hw(H, W, R, S, (sh, sw), (ph, pw))
    total = {"fwd": N * P * Q * K, "dgrad": N * H * W * C, "wgrad": R * S * C * K}[pass_name]
    if idx is None:
        idx = np.arange(total, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int64).ravel()
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < total)
    ch = _chunks(chunk, idx.size)
    t1, t2 = _f32(t1), _f32(t2)
    t, tp, M = _table(lut, M)

    def run(lo, hi):
        out = np.zeros(hi - lo, dtype=np.float32)
        ix, cc = idx[lo:hi], ch[lo:hi]
        lib().orc_conv2d_f32(CONV_PASSES[pass_name], N, H, W, C, K, R, S, sh, sw, ph, pw, _ptr(t1), _ptr(t2),
                             tp, M, E, hi - lo, _ptr(ix), _ptr(cc), _ptr(out))
        return (out,)

    return _threaded(idx.size, threads, run)[0]


# ---------------------------------------------------------------- Conv2D

def conv_out_hw(H, W, R, S, stride, pad):
    sh, sw = stride
    ph, pw = pad
    return (H + 2 * ph - R) // sh + 1, (W + 2 * pw - S) // sw + 1


def _conv(name, shape_out, geomargs, t1, t2, lut, M, idx, E=8, threads=None):
    t1 = _f32(t1)
    t2 = _f32(t2)
    t, tp, M = _table(lut, M)
    if idx is None and not threads:
        total = int(np.prod(shape_out))
        R = np.zeros(total, dtype=np.float64)
        S = np.zeros(total, dtype=np.float64)
        getattr(lib(), name)(*geomargs, _ptr(t1), _ptr(t2), tp, M, E, 0, None,
                             _ptr(R), _ptr(S))
        return R.reshape(shape_out), S.reshape(shape_out)
    whole = idx is None
    if whole:
        idx = np.arange(int(np.prod(shape_out)), dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int64).ravel()

    def run(lo, hi):
        R = np.zeros(hi - lo, dtype=np.float64)
        S = np.zeros(hi - lo, dtype=np.float64)
        ix = idx[lo:hi]
        getattr(lib(), name)(*geomargs, _ptr(t1), _ptr(t2), tp, M, E, hi - lo,
                             _ptr(ix), _ptr(R), _ptr(S))
        return R, S

    R, S = _threaded(idx.size, threads, run)
    return (R.reshape(shape_out), S.reshape(shape_out)) if whole else (R, S)


def conv2d_fwd(x, w, lut, M, stride=(1, 1), pad=(0, 0), idx=None, E=8, threads=None):
    """x: NHWC, w: RSCK. Returns (Y, YS) of shape NPQK (or at flat idx)."""
    N, H, W, C = x.shape
    R, S, C2, K = w.shape
    assert C == C2
    P, Q = conv_out_hw(H, W, R, S, stride, pad)
    g = (N, H, W, C, K, R, S, stride[0], stride[1], pad[0], pad[1])
    return _conv("orc_conv2d_fwd", (N, P, Q, K), g, x, w, lut, M, idx, E, threads)


def conv2d_dgrad(dy, w, x_shape, lut, M, stride=(1, 1), pad=(0, 0), idx=None, E=8, threads=None):
    """dy: NPQK, w: RSCK, x_shape = (N, H, W, C). Returns (dX, dXS)."""
    N, H, W, C = x_shape
    R, S, C2, K = w.shape
    assert C == C2
    P, Q = conv_out_hw(H, W, R, S, stride, pad)
    assert dy.shape == (N, P, Q, K)
    g = (N, H, W, C, K, R, S, stride[0], stride[1], pad[0], pad[1])
    return _conv("orc_conv2d_dgrad", (N, H, W, C), g, dy, w, lut, M, idx, E, threads)


def conv2d_wgrad(x, dy, w_shape, lut, M, stride=(1, 1), pad=(0, 0), idx=None, E=8, threads=None):
    """x: NHWC, dy: NPQK, w_shape = (R, S, C, K). Returns (dW, dWS)."""
    N, H, W, C = x.shape
    R, S, C2, K = w_shape
    assert C == C2
    P, Q = conv_out_hw(H, W, R, S, stride, pad)
    assert dy.shape == (N, P, Q, K)
    g = (N, H, W, C, K, R, S, stride[0], stride[1], pad[0], pad[1])
    return _conv("orc_conv2d_wgrad", (R, S, C, K), g, x, dy, lut, M, idx, E, threads)
