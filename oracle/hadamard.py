"""Randomized Walsh-Hadamard transform (oracle side; test infrastructure).

[arXiv abstract] item (i) and [ICLR abstract]: each tile is rotated by a
randomized Hadamard (Walsh-Hadamard) transform that makes its coordinates close
to Gaussian.  Readings (pages silent): Sylvester ("natural") ordering
H[i][j] = (-1)^popcount(i & j); signs applied before H; orthonormal scaling
1/sqrt(n).  The OrbitQuant README on the same pages describes its own rotation
with the same ingredients (Rademacher signs, block fast WHT, orthonormal
scaling), which corroborates this reading.

The transform is an explicit matrix product, not butterflies.
"""

import math

import numpy as np


def _popcount(a):
    a = np.asarray(a, dtype=np.int64).copy()
    c = np.zeros_like(a)
    while np.any(a):
        c += a & 1
        a >>= 1
    return c


def sylvester(n):
    """n x n Hadamard matrix in Sylvester order, entries +-1.0 (float64)."""
    if n <= 0 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    i = np.arange(n)
    parity = _popcount(np.bitwise_and.outer(i, i)) & 1
    return np.where(parity == 0, 1.0, -1.0)


def unnormalized_forward(x, signs):
    """S = H_n (s * x) per tile (rows of x); exact whenever every partial sum
    of the +-x_j fits in 53 bits (true for bf16 and for the fp32 workloads)."""
    n = x.shape[-1]
    return (np.asarray(x, np.float64) * signs) @ sylvester(n)


def inv_sqrt(n):
    """The orthonormal scale factor, as the fp64 value 1 / sqrt(n)."""
    return 1.0 / math.sqrt(n)


def forward(x, signs):
    """y = H_n diag(s) x / sqrt(n)."""
    return unnormalized_forward(x, signs) / math.sqrt(x.shape[-1])


def inverse(y, signs):
    """x = diag(s) H_n y * (1/sqrt(n)); H is symmetric and H H = n I."""
    n = y.shape[-1]
    return signs * ((np.asarray(y, np.float64) @ sylvester(n)) * inv_sqrt(n))
