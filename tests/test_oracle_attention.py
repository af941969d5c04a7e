"""Pins of the attention oracle: cases whose result the definition fixes
without running it (one key, equal scores, tau = 0, a dominant key), key
order, and a brute-force sum with math.fsum on a tiny case."""

import math

import numpy as np

from oracle.attention import attention


def test_one_key_returns_its_value():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.allclose(attention(q, k, v, 0.7), np.repeat(v, 3, axis=0), rtol=0, atol=1e-15)


def test_equal_scores_and_zero_scale_average_the_values():
    rng = np.random.default_rng(2)
    q, v = rng.standard_normal((4, 8)), rng.standard_normal((5, 8))
    k = np.repeat(rng.standard_normal((1, 8)), 5, axis=0)      # every key the same
    mean = v.mean(axis=0)
    assert np.allclose(attention(q, k, v, 1.3), mean, rtol=0, atol=1e-14)
    k2 = rng.standard_normal((5, 8))
    assert np.allclose(attention(q, k2, v, 0.0), mean, rtol=0, atol=1e-14)


def test_dominant_key_and_key_order():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 8))
    k = rng.standard_normal((6, 8)) * 0.01
    k[4] = q.sum(axis=0) * 10.0          # far the largest score for both queries
    v = rng.standard_normal((6, 8))
    out = attention(q, k, v, 5.0)
    assert np.allclose(out, np.repeat(v[4:5], 2, axis=0), rtol=0, atol=1e-9)
    perm = rng.permutation(6)
    k3, v3 = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    assert np.allclose(attention(q, k3, v3, 0.4), attention(q, k3[perm], v3[perm], 0.4),
                       rtol=0, atol=1e-14)


def test_brute_force_tiny_case():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((2, 4)), rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    tau = 0.5
    out = attention(q, k, v, tau)
    for j in range(2):
        w = [math.exp(tau * math.fsum(q[j, i] * k[t, i] for i in range(4))) for t in range(3)]
        z = math.fsum(w)
        for d in range(4):
            ref = math.fsum(w[t] * v[t, d] for t in range(3)) / z
            assert abs(out[j, d] - ref) <= 1e-14 * max(1.0, abs(ref))
