"""Helpers shared by the GPU parity tests: host<->device transfer and the
comparison rules (indices bit-exact except at oracle near-ties, decoded values
within 1e-5 * Delta, Rice results exact on matching tiles)."""

import numpy as np
import torch

from oracle import codec, rice

NEAR_TIE = 1e-6          # oracle margin below which a block counts as a near-tie
NEAR_TIE_CAP = 1e-5      # largest allowed fraction of excused blocks


def bf16_device(bits, shape=None):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    if shape is not None:
        t = t.reshape(shape)
    return t.cuda()


def f32_device(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def u32(t):
    return host(t).view(np.uint32)


def bf16_host_bits(t):
    return host(t.view(torch.int16)).view(np.uint16)


def tile_rows(gpu_array, n, tiles=None):
    a = np.asarray(gpu_array).reshape(-1, n)
    return a if tiles is None else a[tiles]


def compare_indices(g_idx, g_coset, ora, lattice, n, label=""):
    """Block-level comparison.  Returns (mismatch blocks, near-tie blocks,
    total blocks, tiles whose indices all match)."""
    d = codec.DIM[lattice]
    T = ora["idx"].shape[0]
    gi = np.asarray(g_idx, np.int64).reshape(T, n // d, d)
    oi = ora["idx"].reshape(T, n // d, d)
    bad = np.any(gi != oi, axis=-1)
    if codec.coset_bits_per_tile(lattice, n):
        gc = codec.unpack_cosets(np.asarray(g_coset).reshape(T, -1).astype(np.uint32), lattice, n)
        oc = codec.unpack_cosets(ora["coset"], lattice, n)
        bad |= gc != oc
    near = ora["margin"] < NEAR_TIE
    assert np.all(near[bad]), "%s: %d index mismatches outside near-ties" % (label, np.sum(bad & ~near))
    assert bad.sum() <= NEAR_TIE_CAP * bad.size, "%s: too many near-tie mismatches" % label
    tiles_ok = ~np.any(bad, axis=1)
    return int(bad.sum()), int(near.sum()), int(bad.size), tiles_ok


def compare_decoded(g_vals, o_round, o_raw, scale, out_bf16, exact, label=""):
    """|gpu - oracle fp64| <= 1e-5 * Delta plus the output rounding's own
    error bound at the oracle value: half an ulp of bf16 or fp32, and below
    the smallest normal the flush to zero of bf16 (up to 2^-126) or fp32's
    subnormal spacing (2^-150); `exact` additionally demands bit equality
    with the identically rounded oracle value."""
    g = np.asarray(g_vals, np.float64)
    raw = np.asarray(o_raw, np.float64)
    tol = 1e-5 * np.asarray(scale, np.float64)[:, None]
    if out_bf16:
        rnd = np.where(np.abs(raw) < 2.0 ** -126, 2.0 ** -126, 0.5 * np.abs(raw) * 2.0 ** -7)
    else:
        rnd = np.maximum(0.5 * np.abs(raw) * 2.0 ** -23, 2.0 ** -150)
    tol = tol + rnd
    err = np.abs(g - raw)
    assert np.all(err <= tol), "%s: max err / Delta %.3g" % (
        label, np.max(err / np.asarray(scale)[:, None]))
    if exact:
        o = np.asarray(o_round, np.float64)
        assert np.array_equal(g, o), "%s: %d values differ" % (label, int(np.sum(g != o)))


def oracle_decode_like_gpu(idx, coset, scale, lattice, n, seed, out_bf16,
                           dither_seed=None, dither_base=0):
    """Oracle decode of the given (oracle) indices: (value rounded like the
    output, unrounded fp64 value)."""
    T = np.asarray(idx).size // n
    x = codec.decode(np.asarray(idx, np.int64).reshape(T, n),
                     np.asarray(coset).reshape(T, -1).astype(np.uint32) if coset is not None
                     else np.zeros((T, 0), np.uint32),
                     np.asarray(scale, np.float64), lattice, n, seed,
                     dither_seed=dither_seed, dither_base=dither_base)
    if out_bf16:
        return codec.bf16_rne(x), x
    return x.astype(np.float32).astype(np.float64), x


def rice_pack_oracle(idx, coset_words, lattice, n):
    return rice.pack(np.asarray(idx, np.int64), coset_words,
                     codec.coset_bits_per_tile(lattice, n))
