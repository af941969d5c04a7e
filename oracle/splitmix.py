"""Counter-based random numbers the method draws (oracle side; test infrastructure).

The pages call the Hadamard transform "randomized" ([arXiv abstract], item (i))
and ask for a seeded subtractive dither on the KV path ([ICLR abstract]) but
name no generator.  Reading: both are drawn from the SplitMix64 output function
(G. L. Steele, D. Lea, C. H. Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014), used as a stateless hash of a 64-bit counter key:

    mix(k) = first SplitMix64 output from state k
           = f(k + 0x9E3779B97F4A7C15), where
    f(z):  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
           z ^= z >> 27; z *= 0x94D049BB133111EB;
           z ^= z >> 31            (all arithmetic modulo 2^64)

The HIP library implements the same published function independently.
"""

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MUL1 = np.uint64(0xBF58476D1CE4E5B9)
_MUL2 = np.uint64(0x94D049BB133111EB)


def mix(key):
    """SplitMix64 output for state `key` (uint64 array in, uint64 array out)."""
    z = np.asarray(key, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z + _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _MUL1
        z = (z ^ (z >> np.uint64(27))) * _MUL2
    return z ^ (z >> np.uint64(31))


def rht_signs(seed, n):
    """Random sign vector s of length n for the randomized Hadamard transform.

    Reading (pages silent): s_j = -1 when bit 63 of mix((seed << 32) xor j) is
    set, else +1; one vector per call, shared by every tile of the call.
    `seed` < 2^32.
    """
    if not (0 <= int(seed) < 2**32):
        raise ValueError("rht seed must fit in 32 bits")
    j = np.arange(n, dtype=np.uint64)
    key = (np.uint64(seed) << np.uint64(32)) ^ j
    top = mix(key) >> np.uint64(63)
    return np.where(top == 1, -1.0, 1.0)


def dither_box(seed, vectors, n):
    """Uniform box samples w in [-1, 1)^n for the KV subtractive dither.

    Reading (pages silent on the sampler): for vector index v and coordinate i,
    w = 2^-23 * (mix((seed << 40) xor ((v << 8) | i)) >> 40) - 1, i.e. 24
    random bits mapped onto a 2^-23 grid, exact in fp32 and fp64.  `seed` <
    2^24, v < 2^32, i < 256.  Returns float64 of shape (len(vectors), n).
    """
    if not (0 <= int(seed) < 2**24):
        raise ValueError("dither seed must fit in 24 bits")
    v = np.asarray(vectors, dtype=np.uint64).reshape(-1, 1)
    if v.size and int(v.max()) >= 2**32:
        raise ValueError("dither vector index must fit in 32 bits")
    if n > 256:
        raise ValueError("dither coordinate index must fit in 8 bits")
    i = np.arange(n, dtype=np.uint64).reshape(1, -1)
    key = (np.uint64(seed) << np.uint64(40)) ^ ((v << np.uint64(8)) | i)
    bits24 = mix(key) >> np.uint64(40)
    return bits24.astype(np.float64) * 2.0**-23 - 1.0
