"""Pins for the oracle's counter hash and Hadamard transform (CPU)."""

import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import codec, hadamard, splitmix
import workloads

GAMMA = 0x9E3779B97F4A7C15


def test_splitmix64_known_answers(golden):
    # output index i from initial state s is mix(s + i*gamma)
    for line in golden("splitmix64_vectors.txt"):
        s, i, out = (int(t) for t in line.split())
        key = (s + i * GAMMA) % 2**64
        assert int(splitmix.mix(np.uint64(key))) == out


def test_rht_signs_balanced_and_seeded():
    a = splitmix.rht_signs(1, 256)
    b = splitmix.rht_signs(1, 256)
    c = splitmix.rht_signs(2, 256)
    assert set(np.unique(a)) <= {-1.0, 1.0}
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    big = np.concatenate([splitmix.rht_signs(s, 256) for s in range(64)])
    # fraction of -1 within 5 sigma of 1/2
    frac = np.mean(big < 0)
    assert abs(frac - 0.5) < 5 * math.sqrt(0.25 / big.size)
    # the first n signs do not depend on n (prefix property of the key layout)
    assert np.array_equal(splitmix.rht_signs(7, 128), splitmix.rht_signs(7, 256)[:128])


def test_rht_signs_regression(golden):
    # frozen first 64 signs for seeds 0 and 1 (written by tests/golden/make_golden.py)
    for line in golden("rht_signs.txt"):
        seed, bits = line.split()
        s = splitmix.rht_signs(int(seed), 64)
        assert "".join("1" if v < 0 else "0" for v in s) == bits


def test_dither_box_grid_range_moments():
    w = splitmix.dither_box(2, np.arange(4096), 128)
    assert w.min() >= -1.0 and w.max() < 1.0
    # every value sits on the 2^-23 grid
    assert np.all((w + 1.0) * 2**23 == np.rint((w + 1.0) * 2**23))
    assert abs(w.mean()) < 5 * math.sqrt(1 / 3 / w.size)
    assert abs(np.mean(w * w) - 1 / 3) < 0.005
    # neighbouring keys give unrelated values
    w2 = splitmix.dither_box(3, np.arange(4096), 128)
    assert abs(np.corrcoef(w.ravel(), w2.ravel())[0, 1]) < 0.01


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_sylvester_matches_scipy_and_recursion(n):
    H = hadamard.sylvester(n)
    assert np.array_equal(H, scipy.linalg.hadamard(n).astype(np.float64))
    # Sylvester's recursion H_2n = [[H, H], [H, -H]]
    if n >= 2:
        h = hadamard.sylvester(n // 2)
        assert np.array_equal(H, np.block([[h, h], [h, -h]]))
    assert np.array_equal(H @ H.T, n * np.eye(n))


def test_rht_orthonormal_and_invertible():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 256))
    s = splitmix.rht_signs(9, 256)
    y = hadamard.forward(x, s)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(hadamard.inverse(y, s), x, atol=1e-13)
    # a single nonzero entry spreads to equal magnitudes (a plain rotation would not)
    e = np.zeros((1, 256)); e[0, 3] = 1.0
    assert np.allclose(np.abs(hadamard.forward(e, s)), 1 / 16)


def test_unnormalized_forward_exact_on_bf16_tiles():
    # exact rational arithmetic on a few tiles of the outlier-laden bf16 layer
    x = workloads.bf16_bits_to_f64(workloads.llama_matrix(1, shape=(4, 4096)))
    X = codec.tiles(x, 256)[:6]
    s = splitmix.rht_signs(0, 256)
    S = hadamard.unnormalized_forward(X, s)
    H = hadamard.sylvester(256).astype(int)
    for t in range(X.shape[0]):
        v = [Fraction(float(a)) * int(b) for a, b in zip(X[t], s)]
        for i in range(0, 256, 37):
            exact = sum(int(H[i, j]) * v[j] for j in range(256))
            assert Fraction(float(S[t, i])) == exact


def test_signs_are_applied_before_the_hadamard():
    # e_j maps to s_j * H[:, j] / sqrt(n); applying the signs after H would
    # give s * H[:, j] / sqrt(n) instead
    s = splitmix.rht_signs(4, 64)
    H = hadamard.sylvester(64)
    for j in (0, 5, 63):
        e = np.zeros((1, 64)); e[0, j] = 1.0
        assert np.array_equal(hadamard.forward(e, s)[0], s[j] * H[:, j] / 8.0)
    assert not np.array_equal(s * H[:, 5], s[5] * H[:, 5])
