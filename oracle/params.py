"""Seeded parameters of the codec: the random rotation and the QJL sketch.

Test infrastructure (see the package docstring).  fp64 throughout.

The rotation is the random rotation applied before the polar mapping
("TurboQuant: kompresja KV-cache w LLM 6 razy", section "Zasada dzialania
PolarQuant": the vector is rotated at random, then mapped to polar
coordinates).  The pages name no distribution; the reading taken here is a
Haar-distributed orthogonal matrix: the Q factor of a QR decomposition of a
matrix of i.i.d. standard normals, with the columns' signs fixed so that R has
a positive diagonal (that makes Q unique and Haar).

The sketch is the random projection of the Quantized Johnson-Lindenstrauss
step (same page, section "Kompensacja bledow przez QJL"; and
"TurboQuant: optimizacion de memoria para KV caches", section "Arquitectura
del Sistema").  Reading: i.i.d. N(0, 1) entries, which is what makes the
sqrt(pi/2)/m scaled sign estimator unbiased.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast Splittable
Pseudorandom Number Generators", OOPSLA 2014; the 64-bit finaliser constants
are the published ones from Vigna's reference splitmix64.c), which is a
counter-based generator: output n of a stream seeded with s is mix(s + n*gamma).
Stream k of a cache seed is seeded with mix(seed + (k+1)*gamma).
Uniform doubles take the top 53 bits.  Normals use the Box-Muller transform
on consecutive uniform pairs (u1, u2): sqrt(-2 ln(1-u1)) * (cos 2 pi u2,
sin 2 pi u2), filled row-major.  Stream 0 fills the d x d Gaussian matrix of
the rotation, stream 1 the m_max x d sketch.
"""

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1

STREAM_ROTATION = 0
STREAM_SKETCH = 1
STREAM_HADAMARD_SIGNS = 2


def _mix_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def splitmix64(seed: int, n: int) -> list:
    """First n outputs of SplitMix64 seeded with ``seed`` (Python ints)."""
    return [_mix_int(seed + (i + 1) * GAMMA) for i in range(n)]


def _mix_array(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def stream_seed(seed: int, stream: int) -> int:
    """Seed of stream ``stream`` derived from the cache seed."""
    return _mix_int(seed + (stream + 1) * GAMMA)


def raw_stream(seed: int, stream: int, n: int) -> np.ndarray:
    """n uint64 outputs of stream ``stream`` (vectorised SplitMix64)."""
    s = stream_seed(seed, stream)
    idx = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        x = np.uint64(s) + idx * np.uint64(GAMMA)
        return _mix_array(x)


def uniforms(seed: int, stream: int, n: int) -> np.ndarray:
    """n doubles in [0, 1): top 53 bits of each output times 2^-53."""
    u = raw_stream(seed, stream, n)
    return (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def box_muller(u1: np.ndarray, u2: np.ndarray):
    """Standard normal pair from two uniforms in [0, 1)."""
    rad = np.sqrt(-2.0 * np.log1p(-u1))
    ang = 2.0 * np.pi * u2
    return rad * np.cos(ang), rad * np.sin(ang)


def normals(seed: int, stream: int, n: int) -> np.ndarray:
    """n standard normals of a stream, Box-Muller over consecutive pairs."""
    npair = (n + 1) // 2
    u = uniforms(seed, stream, 2 * npair)
    z0, z1 = box_muller(u[0::2], u[1::2])
    out = np.empty(2 * npair)
    out[0::2] = z0
    out[1::2] = z1
    return out[:n]


def rotation(d: int, seed: int) -> np.ndarray:
    """Haar rotation Pi (d x d, fp64); the codec rotates with y = Pi @ x."""
    g = normals(seed, STREAM_ROTATION, d * d).reshape(d, d)
    q, r = np.linalg.qr(g)
    sgn = np.where(np.diag(r) < 0.0, -1.0, 1.0)
    return q * sgn[None, :]


def sketch(m_max: int, d: int, seed: int) -> np.ndarray:
    """QJL sketch S (m_max x d, fp64); a format with m signs uses rows [0, m)."""
    return normals(seed, STREAM_SKETCH, m_max * d).reshape(m_max, d)


def hadamard_rotation(d: int, seed: int) -> np.ndarray:
    """Randomized Hadamard rotation (the fast alternative to a dense Haar
    rotation, for the ablation): Pi = H_d diag(s) / sqrt(d) with H_d the
    Sylvester-Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]])
    and s_i = +-1 from the top bit of output i of SplitMix64 stream 2 of the
    seed.  d must be a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    top = raw_stream(seed, STREAM_HADAMARD_SIGNS, d) >> np.uint64(63)
    s = np.where(top == np.uint64(1), -1.0, 1.0)
    return h * s[None, :] / np.sqrt(d)
