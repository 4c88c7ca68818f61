"""The seeded random orthogonal (JL) rotation of the residual.

What this module computes: one d x d orthogonal matrix Pi per cache, built
deterministically from the cache's rotation seed, that maps each residual row
into the basis where it is quantised (and back, by its transpose).  Sources:
"A JoLT for the KV cache" (arXiv 2607.12550v4 summary), §1 and §3 (seeded
feature-axis rotation common to all cells, rebuilt by the decoder); the
gist.science summaries, section "JL-Geroteerd Residu" (decoding undoes the
rotation).

Reading taken (the pages name no distribution or generator): Pi is a
Haar-distributed d x d orthogonal matrix obtained as the QR factor of a
Gaussian matrix with the signs of R's diagonal moved into Q (Mezzadri 2007,
"How to generate random matrices from the classical compact groups").  The
Gaussian entries come from SplitMix64 (Steele, Lea and Flood 2014) seeded with
the cache's rotation seed: each 64-bit output x gives the uniform
u = ((x >> 11) + 0.5) * 2^-53 in (0, 1); consecutive uniforms (u1, u2) give two
normals by the Box-Muller transform, sqrt(-2 ln u1) * (cos 2 pi u2, sin 2 pi u2),
filling the matrix row by row.  A residual row r (length d) is stored as
r' = r Pi and decoded as r = r' Pi^T.
"""
import numpy as np

_M64 = (1 << 64) - 1


def splitmix64(seed, n):
    """First n outputs of SplitMix64 from ``seed`` (Python ints)."""
    out = []
    state = seed & _M64
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) & _M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
        out.append(z ^ (z >> 31))
    return out


def splitmix64_array(seed, n):
    """The same n outputs as splitmix64, computed as an array: output i is the
    mixing function of the state seed + (i + 1) * 0x9E3779B97F4A7C15
    (mod 2^64), uint64 arithmetic wrapping as the generator's does."""
    with np.errstate(over="ignore"):
        st = np.uint64(seed & _M64) + (np.arange(1, n + 1, dtype=np.uint64) *
                                        np.uint64(0x9E3779B97F4A7C15))
        z = (st ^ (st >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def uniforms(seed, n):
    xs = splitmix64_array(seed, n)
    return ((xs >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def gaussians(seed, n):
    """First n standard normals of the seeded stream: consecutive uniform
    pairs (u1, u2) -> sqrt(-2 ln u1) (cos 2 pi u2, sin 2 pi u2)."""
    u = uniforms(seed, n + (n & 1))
    u1, u2 = u[0::2], u[1::2]
    rad = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(u.shape[0])
    z[0::2] = rad * np.cos(2.0 * np.pi * u2)
    z[1::2] = rad * np.sin(2.0 * np.pi * u2)
    return z[:n]


def gaussian_matrix(seed, d):
    return gaussians(seed, d * d).reshape(d, d)


def rotation(seed, d):
    """Pi (d x d, float64): Q of the QR factorisation of the seeded Gaussian
    matrix, columns multiplied by sign(diag R)."""
    Z = gaussian_matrix(seed, d)
    Q, R = np.linalg.qr(Z)
    return Q * np.where(np.diag(R) >= 0.0, 1.0, -1.0)


def rotate(rows, Pi):
    return rows @ Pi


def unrotate(rows, Pi):
    return rows @ Pi.T
