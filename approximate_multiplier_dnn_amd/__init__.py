"""Python binding of the LUT-based approximate-multiplier library (libapproxmul.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/approx_mul.h. The names follow
that header. Tensors are torch tensors on the current HIP device (FP32,
contiguous unless a leading dimension is passed); the stream defaults to
torch's current stream.

There is no fallback: importing this package fails if the built library is
missing (run ``__graft_entry__.build()`` or ``approximate_multiplier_dnn_amd/build.py``).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libapproxmul.so")

APPROX_OK = 0
APPROX_EINVAL = -1
APPROX_ENOLUT = -2
APPROX_EUNSUPPORTED = -3
APPROX_EHIP = -4
APPROX_ESCRATCH = -5
APPROX_MAX_GROUP = 4

CONV_PASSES = {"fwd": 0, "dgrad": 1, "wgrad": 2}

MODEL_EXACT = 0
MODEL_MITCHELL = 1

#: every function the C header declares
EXPORTS = (
    "approx_lut_build", "approx_lut_build_from_model", "approx_lut_load", "approx_native_load", "approx_lut_bits",
    "approx_exponent_bits_set", "approx_exponent_bits",
    "approx_gemm", "approx_gemm_noalloc", "approx_gemm_noalloc_max_bytes", "approx_gemm_grouped",
    "approx_gemm_strided_batched", "approx_gemm_batched",
    "approx_conv2d_fwd", "approx_conv2d_dgrad", "approx_conv2d_wgrad",
    "approx_gemm_chunks", "approx_conv2d_chunks",
    "approx_profile_enable", "approx_profile_read",
    "approx_status_string", "approx_build_id", "approx_release",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; the approximate-multiplier path has no fallback")

_lib = ctypes.CDLL(LIB_PATH)

_i, _ll, _vp = ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p
MUL_FN = ctypes.CFUNCTYPE(ctypes.c_float, ctypes.c_float, ctypes.c_float)
_lib.approx_lut_build.argtypes = [_i, _i, _vp, _vp]
_lib.approx_lut_build_from_model.argtypes = [_i, MUL_FN, _vp]
_lib.approx_lut_load.argtypes = [_vp, _i]
_lib.approx_lut_bits.argtypes = []
_lib.approx_exponent_bits_set.argtypes = [_i]
_lib.approx_exponent_bits.argtypes = []
_lib.approx_gemm.argtypes = [_i] * 5 + [_vp, _i, _vp, _i, _vp, _i, _vp]
_lib.approx_gemm_noalloc.argtypes = [_i] * 5 + [_vp, _i, _vp, _i, _vp, _i, _vp]
_lib.approx_gemm_noalloc_max_bytes.argtypes = []
_lib.approx_gemm_strided_batched.argtypes = [_i] * 5 + [_vp, _i, _ll, _vp, _i, _ll, _vp, _i, _ll, _i, _vp]
_lib.approx_gemm_batched.argtypes = [_i] * 5 + [_vp, _i, _vp, _i, _vp, _i, _i, _vp]
_lib.approx_gemm_grouped.argtypes = [_i] + [_vp] * 12
for _n in ("approx_conv2d_fwd", "approx_conv2d_dgrad", "approx_conv2d_wgrad"):
    getattr(_lib, _n).argtypes = [_i] * 11 + [_vp, _vp, _vp, _vp]
_lib.approx_gemm_chunks.argtypes = [_i] * 6 + [_ll, _vp, _vp, _vp, _vp]
_lib.approx_conv2d_chunks.argtypes = [_i] * 12 + [_ll, _vp, _vp]
_lib.approx_status_string.argtypes = [_i]
_lib.approx_status_string.restype = ctypes.c_char_p
_lib.approx_build_id.argtypes = []
_lib.approx_build_id.restype = ctypes.c_char_p
_lib.approx_release.argtypes = []
_lib.approx_profile_enable.argtypes = [_i]
_lib.approx_profile_read.argtypes = [_vp, _vp]
for _n in EXPORTS:
    if _n not in ("approx_status_string", "approx_build_id", "approx_gemm_noalloc_max_bytes"):
        getattr(_lib, _n).restype = ctypes.c_int
_lib.approx_gemm_noalloc_max_bytes.restype = ctypes.c_longlong


class ApproxError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {approx_status_string(status)} ({status})")
        self.status = status


def lib():
    return _lib


def _check(rc, what):
    if rc != APPROX_OK:
        raise ApproxError(rc, what)
    return rc


def approx_status_string(status):
    return _lib.approx_status_string(int(status)).decode()


def approx_build_id():
    """Stamp of the sources the loaded library was built from."""
    return _lib.approx_build_id().decode()


# ------------------------------------------------------------------ tables

def approx_lut_build(model, M, perturb=None):
    """Table of 4**M uint16 entries (Algorithm 1) for MODEL_EXACT or
    MODEL_MITCHELL, optionally moved by a +/-1 int8 perturbation."""
    out = np.zeros(1 << (2 * M), dtype=np.uint16)
    p = None
    if perturb is not None:
        p = np.ascontiguousarray(perturb, dtype=np.int8)
        if p.size != out.size:
            raise ValueError("perturbation must have 4**M entries")
    _check(_lib.approx_lut_build(int(model), int(M), p.ctypes.data if p is not None else None,
                                 out.ctypes.data), "approx_lut_build")
    return out


def approx_lut_build_from_model(M, mul):
    """Table from a Python model float(float, float) of the multiplier."""
    out = np.zeros(1 << (2 * M), dtype=np.uint16)
    cb = MUL_FN(lambda a, b: float(mul(a, b)))
    _check(_lib.approx_lut_build_from_model(int(M), cb, out.ctypes.data), "approx_lut_build_from_model")
    return out


def approx_lut_load(lut, M):
    t = np.ascontiguousarray(lut, dtype=np.uint16)
    if t.size != (1 << (2 * M)):
        raise ValueError("table must have 4**M entries")
    _check(_lib.approx_lut_load(t.ctypes.data, int(M)), "approx_lut_load")


def approx_native_load():
    """Select the native FP32 multiplier (fused multiply-add) on the current device."""
    _check(_lib.approx_native_load(), "approx_native_load")


def approx_lut_bits():
    return _lib.approx_lut_bits()


def approx_exponent_bits_set(E):
    """Exponent width E (1..8) of the multiplier's format (1, E, M) on the current device."""
    _check(_lib.approx_exponent_bits_set(int(E)), "approx_exponent_bits_set")


def approx_exponent_bits():
    return _lib.approx_exponent_bits()


def approx_release():
    _check(_lib.approx_release(), "approx_release")


def approx_profile_enable(on=True):
    _check(_lib.approx_profile_enable(1 if on else 0), "approx_profile_enable")


def approx_profile_read():
    """(launches, total_ms) of the GEMM kernel since the last read."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(_lib.approx_profile_read(ctypes.byref(n), ctypes.byref(ms)), "approx_profile_read")
    return n.value, ms.value


# ------------------------------------------------------------------ compute

def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if t.dtype != torch.float32 or not t.is_cuda:
        raise TypeError("expected a float32 tensor on the GPU")
    return t.data_ptr()


def approx_gemm(transA, transB, m, n, k, A, lda, B, ldb, C, ldc, stream=None):
    """C (m x n, leading dimension ldc) = op(A) op(B) with approximate products."""
    return _check(_lib.approx_gemm(int(transA), int(transB), int(m), int(n), int(k), _ptr(A), int(lda),
                                   _ptr(B), int(ldb), _ptr(C), int(ldc), _stream(stream)), "approx_gemm")


def approx_gemm_grouped(calls, stream=None):
    """Independent GEMMs in one call: `calls` holds 1 .. APPROX_MAX_GROUP
    tuples (transA, transB, m, n, k, A, lda, B, ldb, C, ldc), approx_gemm's
    arguments; each C gets the bits approx_gemm would give it."""
    calls = list(calls)
    cnt = len(calls)
    if not 1 <= cnt <= APPROX_MAX_GROUP:
        return _check(APPROX_EINVAL, "approx_gemm_grouped")
    ints = [(ctypes.c_int * cnt)(*(int(c[f]) for c in calls)) for f in (0, 1, 2, 3, 4, 6, 8, 10)]
    ptrs = [(ctypes.c_void_p * cnt)(*(_ptr(c[f]) for c in calls)) for f in (5, 7, 9)]
    tA, tB, m, n, k, lda, ldb, ldc = ints
    A, B, C = ptrs
    return _check(_lib.approx_gemm_grouped(cnt, tA, tB, m, n, k, A, lda, B, ldb, C, ldc, _stream(stream)),
                  "approx_gemm_grouped")


def approx_gemm_chunks(transA, transB, m, n, k, batch, b, i, j):
    """Summation chunk length of each output (b[t], i[t], j[t]) of a GEMM
    call with these sizes on the current device (k: one chunk)."""
    bb = np.ascontiguousarray(np.broadcast_to(np.asarray(b, dtype=np.int32), np.shape(i)), dtype=np.int32).ravel()
    ii = np.ascontiguousarray(i, dtype=np.int32).ravel()
    jj = np.ascontiguousarray(j, dtype=np.int32).ravel()
    assert ii.shape == jj.shape == bb.shape
    out = np.zeros(ii.size, dtype=np.int64)
    _check(_lib.approx_gemm_chunks(int(transA), int(transB), int(m), int(n), int(k), int(batch), ii.size,
                                   bb.ctypes.data, ii.ctypes.data, jj.ctypes.data, out.ctypes.data),
           "approx_gemm_chunks")
    return out


def approx_conv2d_chunks(pass_name, N, H, W, C, K, R, S, stride, pad, idx):
    """Summation chunk length of the outputs at flat indices idx of a Conv2D
    pass ("fwd", "dgrad" or "wgrad") on the current device."""
    ix = np.ascontiguousarray(idx, dtype=np.int64).ravel()
    out = np.zeros(ix.size, dtype=np.int64)
    _check(_lib.approx_conv2d_chunks(CONV_PASSES[pass_name], int(N), int(H), int(W), int(C), int(K), int(R),
                                     int(S), int(stride[0]), int(stride[1]), int(pad[0]), int(pad[1]), ix.size,
                                     ix.ctypes.data, out.ctypes.data), "approx_conv2d_chunks")
    return out


def approx_gemm_noalloc(transA, transB, m, n, k, A, lda, B, ldb, C, ldc, stream=None):
    """approx_gemm without any allocation (fixed per-device scratch)."""
    return _check(_lib.approx_gemm_noalloc(int(transA), int(transB), int(m), int(n), int(k), _ptr(A), int(lda),
                                           _ptr(B), int(ldb), _ptr(C), int(ldc), _stream(stream)),
                  "approx_gemm_noalloc")


def approx_gemm_noalloc_max_bytes():
    return int(_lib.approx_gemm_noalloc_max_bytes())


def approx_gemm_strided_batched(transA, transB, m, n, k, A, lda, strideA, B, ldb, strideB, C, ldc, strideC,
                                batch, stream=None):
    return _check(_lib.approx_gemm_strided_batched(
        int(transA), int(transB), int(m), int(n), int(k), _ptr(A), int(lda), int(strideA), _ptr(B), int(ldb),
        int(strideB), _ptr(C), int(ldc), int(strideC), int(batch), _stream(stream)), "approx_gemm_strided_batched")


def approx_gemm_batched(transA, transB, m, n, k, A_ptrs, lda, B_ptrs, ldb, C_ptrs, ldc, batch, stream=None):
    """Batched GEMM by device pointer arrays (int64 tensors of data pointers on the GPU)."""
    def arr(t):
        if isinstance(t, int):
            return t
        import torch
        if t.dtype != torch.int64 or not t.is_cuda or t.numel() < batch:
            raise TypeError("pointer arrays must be int64 GPU tensors with one entry per batch")
        return t.data_ptr()
    return _check(_lib.approx_gemm_batched(int(transA), int(transB), int(m), int(n), int(k), arr(A_ptrs), int(lda),
                                           arr(B_ptrs), int(ldb), arr(C_ptrs), int(ldc), int(batch),
                                           _stream(stream)), "approx_gemm_batched")


def pointer_array(tensors_or_ptrs, device="cuda"):
    """int64 device tensor holding the data pointers of the given tensors."""
    import torch
    ptrs = [t if isinstance(t, int) else t.data_ptr() for t in tensors_or_ptrs]
    return torch.tensor(ptrs, dtype=torch.int64, device=device)


def _conv_call(name, N, H, W, C, K, R, S, stride, pad, t1, t2, out, stream):
    fn = getattr(_lib, name)
    return _check(fn(int(N), int(H), int(W), int(C), int(K), int(R), int(S), int(stride[0]), int(stride[1]),
                     int(pad[0]), int(pad[1]), _ptr(t1), _ptr(t2), _ptr(out), _stream(stream)), name)


def approx_conv2d_fwd(N, H, W, C, K, R, S, stride, pad, x, w, y, stream=None):
    return _conv_call("approx_conv2d_fwd", N, H, W, C, K, R, S, stride, pad, x, w, y, stream)


def approx_conv2d_dgrad(N, H, W, C, K, R, S, stride, pad, dy, w, dx, stream=None):
    return _conv_call("approx_conv2d_dgrad", N, H, W, C, K, R, S, stride, pad, dy, w, dx, stream)


def approx_conv2d_wgrad(N, H, W, C, K, R, S, stride, pad, x, dy, dw, stream=None):
    return _conv_call("approx_conv2d_wgrad", N, H, W, C, K, R, S, stride, pad, x, dy, dw, stream)


# ------------------------------------------------------------------ tensor helpers

def gemm(A, B, transA=False, transB=False, out=None, stream=None):
    """op(A) @ op(B) for contiguous 2-D tensors; allocates the output."""
    import torch
    m = A.shape[1] if transA else A.shape[0]
    k = A.shape[0] if transA else A.shape[1]
    n = B.shape[0] if transB else B.shape[1]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=A.device)
    approx_gemm(transA, transB, m, n, k, A, A.stride(0), B, B.stride(0), out, out.stride(0), stream)
    return out


def conv_out_hw(H, W, R, S, stride, pad):
    return (H + 2 * pad[0] - R) // stride[0] + 1, (W + 2 * pad[1] - S) // stride[1] + 1


def conv2d_fwd(x, w, stride=(1, 1), pad=(0, 0), stream=None):
    """x NHWC, w RSCK -> y NPQK."""
    import torch
    N, H, W, C = x.shape
    R, S, _, K = w.shape
    P, Q = conv_out_hw(H, W, R, S, stride, pad)
    y = torch.empty((N, P, Q, K), dtype=torch.float32, device=x.device)
    approx_conv2d_fwd(N, H, W, C, K, R, S, stride, pad, x, w, y, stream)
    return y


def conv2d_dgrad(dy, w, x_shape, stride=(1, 1), pad=(0, 0), stream=None):
    import torch
    N, H, W, C = x_shape
    R, S, _, K = w.shape
    dx = torch.empty((N, H, W, C), dtype=torch.float32, device=dy.device)
    approx_conv2d_dgrad(N, H, W, C, K, R, S, stride, pad, dy, w, dx, stream)
    return dx


def conv2d_wgrad(x, dy, w_shape, stride=(1, 1), pad=(0, 0), stream=None):
    import torch
    N, H, W, C = x.shape
    R, S, _, K = w_shape
    dw = torch.empty((R, S, C, K), dtype=torch.float32, device=x.device)
    approx_conv2d_wgrad(N, H, W, C, K, R, S, stride, pad, x, dy, dw, stream)
    return dw
