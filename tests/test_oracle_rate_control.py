"""Pins for the oracle's per-tile rate control (reading R7 in oracle/codec.py):
the bisection against an exhaustive scan of the same bf16 window, the
chosen scales re-encoded through the plain explicit-scale path, and the
special cases (zero and non-finite tiles, budgets no scale can meet)."""

import math

import numpy as np

from oracle import codec, hadamard, rice, splitmix


def _tiles(seed, T, n, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, n)) * 0.02
    if outliers:
        x[:, 3] *= 60.0
    bits = (x.astype(np.float32).view(np.uint32) + 0x7FFF +
            ((x.astype(np.float32).view(np.uint32) >> 16) & 1)) >> 16
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)   # bf16 values


def _fits(X, S, lattice, bps, codes):
    """Feasibility of one bf16 pattern per tile, through the explicit-scale
    encode (the plain path) rather than the search's own helper."""
    n = X.shape[1]
    delta = codec.bf16_from_bits(np.asarray(codes, np.uint16))
    u = codec.quantizer_input(S, delta, lattice)
    z, c, _ = codec.nearest(u, lattice)
    idx = codec.strip(z, c, lattice)
    ok = ~np.any((idx < -128) | (idx > 127), axis=1)
    _, tb = rice.tile_bits(np.clip(idx, -128, 127), codec.coset_bits_per_tile(lattice, n))
    return ok & (tb <= math.floor(bps * n))


def test_bisection_matches_exhaustive_scan():
    for lattice, n, bps in (("E8", 64, 3.0), ("Z", 64, 4.0), ("A2", 64, 3.5)):
        X = _tiles(7, 24, n)
        signs = splitmix.rht_signs(5, n)
        S = hadamard.unnormalized_forward(X, signs)
        got = codec.rate_controlled_scale(X, S, lattice, bps)
        a = codec.bf16_bits(codec.auto_scale(X, lattice, bps)).astype(np.int64)
        lo = np.maximum(a - 1024, 0x0080)
        hi = np.minimum(a + 1024, 0x7F7F)
        # feasibility of every pattern in the widest window, tile by tile
        codes = np.arange(int(lo.min()), int(hi.max()) + 1)
        F = np.stack([_fits(X, S, lattice, bps, np.full(len(X), c)) for c in codes], axis=1)
        gb = codec.bf16_bits(got).astype(np.int64)
        upsets = 0
        for t in range(len(X)):
            w = (codes > lo[t]) & (codes <= hi[t])          # patterns the search can return
            ft = F[t, w]
            ct = codes[w]
            assert F[t, codes == hi[t]][0], "the window's top is feasible at %g bps" % bps
            first = ct[np.argmax(ft)]
            if np.all(ft[ct >= first]):
                # feasibility is an up-set: bisection finds its least element
                upsets += 1
                assert gb[t] == first, (lattice, t, gb[t], first)
            else:
                # otherwise a crossing: feasible, the pattern below not
                i = int(np.nonzero(codes == gb[t])[0][0])
                assert F[t, i] and not F[t, i - 1], (lattice, t)
        assert upsets >= len(X) // 2


def test_chosen_scales_fit_and_spend_the_budget():
    for lattice, n in (("E8", 256), ("D4", 128), ("Z", 512)):
        X = _tiles(11, 48, n)
        x = X.reshape(8, -1)
        o = codec.encode(x, lattice, n, 4.0, rht_seed=2, rate_control=True)
        # the chosen scales through the explicit-scale path
        e = codec.encode(x, lattice, n, 4.0, rht_seed=2, scale=o["scale"])
        assert np.array_equal(e["idx"], o["idx"]) and np.array_equal(e["tile_bits"], o["tile_bits"])
        assert not e["overflow"].any()
        assert np.all(e["tile_bits"] <= 4 * n)
        # one bf16 step finer breaks the budget or the int8 range
        finer = codec.bf16_from_bits(codec.bf16_bits(o["scale"]).astype(np.uint16) - 1)
        f = codec.encode(x, lattice, n, 4.0, rht_seed=2, scale=finer)
        assert np.all(f["overflow"] | (f["tile_bits"] > 4 * n))
        assert e["tile_bits"].mean() > 0.97 * 4 * n


def test_special_tiles():
    n = 64
    X = _tiles(3, 6, n)
    X[1] = 0.0
    X[2, 5] = np.nan
    S = hadamard.unnormalized_forward(np.nan_to_num(X), splitmix.rht_signs(0, n))
    S[2] = np.nan
    got = codec.rate_controlled_scale(X, S, "E8", 3.0)
    assert got[1] == 1.0                          # an all-zero tile keeps scale 1
    assert np.isnan(got[2])                       # a non-finite tile keeps its automatic scale
    # a budget below n + 4 + coset bits: no scale fits, the tile takes the top of its window
    low = codec.rate_controlled_scale(X[[0, 3]], S[[0, 3]], "E8", 0.5)
    a = codec.bf16_bits(codec.auto_scale(X[[0, 3]], "E8", 0.5)).astype(np.int64)
    assert np.array_equal(codec.bf16_bits(low).astype(np.int64), np.minimum(a + 1024, 0x7F7F))
