"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds random-number generation and workload shapes only: none of
the approximate-multiplication arithmetic. Both the HIP path and the oracle
receive the same bytes from here.

Generator: splitmix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; the constants of S. Vigna's
public-domain splitmix64.c). Draw t of stream ``seed`` is the output function
applied to seed + (t+1) * 0x9E3779B97F4A7C15 (mod 2**64), so any draw can be
computed on its own. Uniform doubles take the top 53 bits; normals use the
Box-Muller transform on two uniform draws (cosine branch only); float32 values
are the float64 results rounded to nearest-even.
"""
import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

#: seed of the +/-1 table perturbation stream
PERTURB_SEED = 0x5EED0008


_CHUNK = 1 << 20


def _draws_into(seed, start, z, tmp, base):
    """z[:] = draws start .. start+len(z)-1 of stream ``seed`` (in place)."""
    n = z.size
    np.add(base[:n], np.uint64(start), out=z)
    with np.errstate(over="ignore"):
        np.multiply(z, _GOLDEN, out=z)
        np.add(z, np.uint64(seed), out=z)
        np.right_shift(z, np.uint64(30), out=tmp[:n])
        np.bitwise_xor(z, tmp[:n], out=z)
        np.multiply(z, _M1, out=z)
        np.right_shift(z, np.uint64(27), out=tmp[:n])
        np.bitwise_xor(z, tmp[:n], out=z)
        np.multiply(z, _M2, out=z)
        np.right_shift(z, np.uint64(31), out=tmp[:n])
        np.bitwise_xor(z, tmp[:n], out=z)


def _chunks(count):
    for s in range(0, count, _CHUNK):
        yield s, min(_CHUNK, count - s)


def _buffers():
    base = np.arange(1, _CHUNK + 1, dtype=np.uint64)
    return np.empty(_CHUNK, np.uint64), np.empty(_CHUNK, np.uint64), base


def splitmix64(seed, count, start=0):
    """Draws start .. start+count-1 of stream ``seed`` as uint64."""
    out = np.empty(count, dtype=np.uint64)
    z, tmp, base = _buffers()
    for s, n in _chunks(count):
        _draws_into(seed, start + s, z[:n], tmp, base)
        out[s:s + n] = z[:n]
    return out


def uniform01(seed, count):
    """float64 in [0, 1): the top 53 bits of each draw."""
    out = np.empty(count, dtype=np.float64)
    z, tmp, base = _buffers()
    for s, n in _chunks(count):
        _draws_into(seed, s, z[:n], tmp, base)
        np.right_shift(z[:n], np.uint64(11), out=z[:n])
        np.multiply(z[:n], 2.0 ** -53, out=out[s:s + n], casting="unsafe")
    return out


def normal(seed, shape, std=1.0, mean=0.0):
    """float32 N(mean, std**2) of the given shape (Box-Muller, cosine branch):
    value t uses uniform draws 2t and 2t+1."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    z, tmp, base = _buffers()
    u = np.empty(_CHUNK, np.float64)
    half = _CHUNK // 2
    for s in range(0, n, half):
        c = min(half, n - s)
        _draws_into(seed, 2 * s, z[:2 * c], tmp, base)
        np.right_shift(z[:2 * c], np.uint64(11), out=z[:2 * c])
        np.multiply(z[:2 * c], 2.0 ** -53, out=u[:2 * c], casting="unsafe")
        u1 = u[0:2 * c:2]
        u2 = u[1:2 * c:2]
        r = np.sqrt(-2.0 * np.log1p(-u1))
        v = r * np.cos(2.0 * np.pi * u2)
        out[s:s + c] = (mean + std * v).astype(np.float32)
    return out.reshape(shape)


def uniform(seed, shape, low=0.0, high=1.0):
    """float32 U(low, high) of the given shape."""
    n = int(np.prod(shape))
    u = uniform01(seed, n)
    return (low + (high - low) * u).astype(np.float32).reshape(shape)


def glorot_uniform(seed, fan_in, fan_out):
    """[fan_in x fan_out] weights ~ U(-a, a), a = sqrt(6 / (fan_in + fan_out))."""
    a = np.sqrt(6.0 / (fan_in + fan_out))
    return uniform(seed, (fan_in, fan_out), -a, a)


def he_normal(seed, shape, fan_in):
    """weights ~ N(0, 2 / fan_in) (untruncated)."""
    return normal(seed, shape, std=np.sqrt(2.0 / fan_in))


def pm_one(seed, count):
    """int8 +1 / -1 per draw: +1 when bit 0 of the draw is set."""
    bit = (splitmix64(seed, count) & np.uint64(1)).astype(np.int8)
    return (2 * bit - 1).astype(np.int8)


def tensor_seed(config, tensor_id):
    """Per-tensor seed: 1000 * config + tensor id."""
    return 1000 * config + tensor_id


def special_values():
    """float32 edge values: signed zeros, subnormals, extremes, Inf, NaN."""
    u = np.array([
        0x00000000, 0x80000000,            # +0, -0
        0x00000001, 0x807FFFFF, 0x00400000,  # subnormals
        0x00800000, 0x80800000,            # smallest normals
        0x00FFFFFF, 0x3F800000, 0xBF800000,  # 1, -1
        0x3FC00000, 0x40400000,            # 1.5, 3
        0x7F7FFFFF, 0xFF7FFFFF,            # largest finite
        0x7F000000, 0x1F800000, 0x20000000, 0x5F000000, 0x5F800000,
        0x7F800000, 0xFF800000,            # +-Inf
        0x7FC00000, 0xFFC00001, 0x7F800001,  # NaNs
    ], dtype=np.uint32)
    return u.view(np.float32)
