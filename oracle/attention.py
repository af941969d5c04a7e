"""Attention of one head over a decoded KV cache: the plain definition.

TEST INFRASTRUCTURE ONLY: see the package docstring.

[ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice Quantization
Pipeline ..." (the subtractive dither keeps each cached inner product
unbiased, so the decoded keys and values serve attention directly).  The
pages give no attention procedure; the reading taken here is textbook
softmax attention of one head over the cache, with k_hat and v_hat the
codec's (dithered) decodes:

    out_j = sum_k a_jk v_hat_k,   a_jk = exp(tau q_j . k_hat_k) / sum_k' exp(tau q_j . k_hat_k')

in fp64, the max score subtracted before the exponent (which leaves a_jk
unchanged in exact arithmetic).
"""

import numpy as np


def attention(q, k_hat, v_hat, tau):
    """q (n_q, d), k_hat and v_hat (n_keys, d), tau the score scale (the
    usual 1 / sqrt(d)); returns out (n_q, d) fp64."""
    q = np.asarray(q, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    v_hat = np.asarray(v_hat, np.float64)
    s = tau * (q @ k_hat.T)                       # scores (n_q, n_keys)
    s = s - s.max(axis=1, keepdims=True)
    a = np.exp(s)
    a = a / a.sum(axis=1, keepdims=True)          # softmax over the keys
    return a @ v_hat
