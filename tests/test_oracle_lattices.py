"""Pins for the oracle's nearest-point rules (CPU): exhaustive search, worked
examples, membership, textbook normalized second moments, margins."""

import itertools
import math

import numpy as np
import pytest

from oracle import codec, lattices as L

GRID = 2.0 ** 24
DIMS = {"E8": 8, "D4": 4, "A2": 2, "Z": 1}


def decode_point(u, lat):
    """Decoder output as a point in decision coordinates."""
    if lat == "E8":
        z, c = L.e8_nearest(u)
        return L.e8_point(z, c)
    if lat == "D4":
        return L.d4_nearest(u).astype(float)
    if lat == "A2":
        ab, c = L.a2_nearest(u)
        return ab + 0.5 * c[..., None]
    return L.z_nearest(u).astype(float)


def metric(lat):
    return L.A2_METRIC if lat == "A2" else None


def on_grid(a):
    return np.rint(np.asarray(a) * GRID) / GRID


def adversarial(lat, rng, count):
    """Grid points on or next to decision boundaries."""
    d = DIMS[lat]
    out = []
    # every coordinate at k + 1/2, or at integers, with random signs/offsets
    base = rng.integers(-5, 6, size=(count, d)).astype(float)
    out.append(base + 0.5)
    out.append(base)
    # midpoints between a lattice point and a neighbour, +-0..2 grid steps
    roots = {"E8": L.E8_ROOTS, "D4": L.D4_ROOTS, "A2": L.A2_ROOTS, "Z": L.Z_ROOTS}[lat]
    p = decode_point(on_grid(rng.uniform(-6, 6, size=(count, d))), lat)
    r = roots[rng.integers(0, len(roots), size=count)]
    jitter = rng.integers(-2, 3, size=(count, d)) / GRID
    out.append(p + r / 2 + jitter)
    if lat == "E8":
        deep = np.zeros((count, 8)); deep[np.arange(count), rng.integers(0, 8, count)] = 1.0
        out.append(deep + p)
        # odd-sum integer points (the D8 parity fix must fire)
        odd = rng.integers(-3, 4, size=(count, 8)).astype(float)
        odd[:, 0] += (odd.sum(1) % 2 == 0)
        out.append(odd)
    return np.concatenate(out)


@pytest.mark.parametrize("lat", ["E8", "D4", "A2", "Z"])
def test_worked_examples(golden, lat):
    rows = [r for r in golden("decoder_examples.txt") if r.split("|")[0].strip() == lat]
    assert rows
    for r in rows:
        _, u, p, dist = (t.strip() for t in r.split("|"))
        u = np.array([[float(t) for t in u.split()]])
        p = np.array([[float(t) for t in p.split()]])
        got = decode_point(u, lat)
        assert np.array_equal(got, p), (lat, u, got)
        assert math.isclose(L.sqdist(u - got, metric(lat))[0], float(dist), abs_tol=1e-12)
        assert math.isclose(L.brute_force(u, lat)[0][0], float(dist), abs_tol=1e-12)


@pytest.mark.parametrize("lat", ["E8", "D4", "A2", "Z"])
def test_decoder_equals_exhaustive_search(lat):
    rng = np.random.default_rng(11)
    d = DIMS[lat]
    pts = [on_grid(rng.normal(0, 4, size=(1500, d))),
           on_grid(rng.uniform(-3, 3, size=(1500, d))),
           adversarial(lat, rng, 300)]
    u = np.concatenate(pts)
    p = decode_point(u, lat)
    for lo in range(0, len(u), 250):
        best, cand, dist = L.brute_force(u[lo:lo + 250], lat)
        got = L.sqdist(u[lo:lo + 250] - p[lo:lo + 250], metric(lat))
        # exact arithmetic on the grid: equal distances, not just close
        assert np.array_equal(got, best)


def _member(p, lat):
    if lat == "E8":
        P = 2 * p
        assert np.all(P == np.rint(P))
        par = np.mod(P, 2)
        assert np.all(par == par[..., :1])
        assert np.all(np.mod(P.sum(-1), 4) == 0)
    elif lat == "D4":
        assert np.all(p == np.rint(p)) and np.all(np.mod(p.sum(-1), 2) == 0)
    elif lat == "A2":
        P = 2 * p
        assert np.all(P == np.rint(P))
        assert np.all(np.mod(P[..., 0], 2) == np.mod(P[..., 1], 2))
    else:
        assert np.all(p == np.rint(p))


@pytest.mark.parametrize("lat", ["E8", "D4", "A2", "Z"])
def test_membership_idempotence_translation(lat):
    rng = np.random.default_rng(3)
    d = DIMS[lat]
    u = on_grid(rng.normal(0, 6, size=(20000, d)))
    p = decode_point(u, lat)
    _member(p, lat)
    assert np.array_equal(decode_point(p, lat), p)
    # Q(u + lam) = Q(u) + lam for lattice vectors lam, away from ties
    lam = decode_point(on_grid(rng.normal(0, 10, size=(20000, d))), lat)
    mu = L.margin(u - p, {"E8": L.E8_ROOTS, "D4": L.D4_ROOTS, "A2": L.A2_ROOTS,
                          "Z": L.Z_ROOTS}[lat], metric(lat))
    ok = mu > 0
    assert np.array_equal(decode_point(u + lam, lat)[ok], (p + lam)[ok])


def _e8_vectors_upto_norm4():
    ints = np.array(list(itertools.product(range(-2, 3), repeat=8)), float)
    ints = ints[(ints.sum(1) % 2 == 0)]
    halves = np.array(list(itertools.product((-1.5, -0.5, 0.5, 1.5), repeat=8)))
    halves = halves[np.mod((halves - 0.5).sum(1), 2) == 0]
    v = np.concatenate([ints, halves])
    nn = (v * v).sum(1)
    return v[(nn > 0) & (nn <= 4)]


def test_e8_vector_counts():
    v = _e8_vectors_upto_norm4()
    nn = (v * v).sum(1)
    # E8 theta series: 240 vectors of norm 2, 2160 of norm 4
    assert (nn == 2).sum() == 240 and (nn == 4).sum() == 2160
    assert len(L.E8_ROOTS) == 240
    assert set(map(tuple, L.E8_ROOTS)) == set(map(tuple, v[nn == 2]))


@pytest.mark.parametrize("lat", ["E8", "D4", "A2", "Z"])
def test_margin_is_second_nearest_gap(lat):
    rng = np.random.default_rng(17)
    d = DIMS[lat]
    u = np.concatenate([on_grid(rng.uniform(-3, 3, size=(1500, d))), adversarial(lat, rng, 100)])
    p = decode_point(u, lat)
    roots = {"E8": L.E8_ROOTS, "D4": L.D4_ROOTS, "A2": L.A2_ROOTS, "Z": L.Z_ROOTS}[lat]
    mu = L.margin(u - p, roots, metric(lat))
    d1 = L.sqdist(u - p, metric(lat))
    # brute force over all lattice vectors of (weighted) norm^2 <= 4 around p
    if lat == "E8":
        vec = _e8_vectors_upto_norm4()
    else:
        rng_vals = np.arange(-4, 4.5, 0.5) if lat == "A2" else np.arange(-2, 3)
        cand = np.array(list(itertools.product(rng_vals, repeat=d)), float)
        if lat == "A2":
            cand = cand[np.mod(2 * cand[:, 0], 2) == np.mod(2 * cand[:, 1], 2)]
        if lat == "D4":
            cand = cand[cand.sum(1) % 2 == 0]
        nn = L.sqdist(cand, metric(lat))
        vec = cand[(nn > 0) & (nn <= 4)]
    for lo in range(0, len(u), 100):
        x = (u - p)[lo:lo + 100]
        d2 = L.sqdist(x[:, None, :] - vec[None], metric(lat)).min(1)
        assert np.array_equal(d2 - d1[lo:lo + 100], mu[lo:lo + 100])


def test_exact_ties_follow_the_stated_rules():
    # u exactly halfway between the two cosets' candidates: the coset tie goes
    # to the integer coset; a pure coordinate tie rounds half to even
    u = np.array([[0.25] * 8])            # |u-0|^2 = 0.5 = |u - (1/2)^8|^2
    z, c = L.e8_nearest(u)
    assert c[0] == 0 and np.array_equal(z[0], np.zeros(8))
    w = np.array([[0.25, 0.25]])          # A2: 1/16 + 3/16 both ways
    ab, c = L.a2_nearest(w)
    assert c[0] == 0 and np.array_equal(ab[0], [0, 0])


def nsm(lat, rng, count=1_000_000):
    d = DIMS[lat]
    if lat in ("E8", "D4"):
        u = rng.uniform(0, 2, size=(count, d))
    else:
        u = rng.uniform(0, 1, size=(count, d))     # Z, and A2 in w coordinates
    e = u - decode_point(u, lat)
    m2 = L.sqdist(e, metric(lat)).mean()
    vol = {"E8": 1.0, "D4": 2.0, "A2": math.sqrt(3) / 2, "Z": 1.0}[lat]
    return m2 / (d * vol ** (2.0 / d))


@pytest.mark.parametrize("lat", ["E8", "D4", "A2", "Z"])
def test_normalized_second_moment(golden, lat):
    table = {r.split()[0]: float(r.split()[2]) for r in golden("nsm_textbook.txt")}
    g = nsm(lat, np.random.default_rng(99))
    assert abs(g / table[lat] - 1.0) < 0.005, (lat, g, table[lat])
    # and the oracle's normalisation constant agrees with the volume used here
    assert math.isclose(codec.vol_root(lat) ** DIMS[lat],
                        {"E8": 1.0, "D4": 2.0, "A2": math.sqrt(3) / 2, "Z": 1.0}[lat])


def test_plausible_mistakes_are_caught():
    """A D8 rule that fixes parity on the wrong coordinate, or an E8 rule that
    drops the half-integer coset, must fail the exhaustive comparison."""
    rng = np.random.default_rng(8)
    u = on_grid(rng.uniform(-2, 2, size=(400, 8)))
    best = L.brute_force(u, "E8")[0]

    def wrong_parity(v):
        f = np.rint(v)
        odd = (f.sum(-1) % 2) != 0
        f[odd, 0] += 1.0                 # always the first coordinate
        return f
    a = wrong_parity(u)
    b = wrong_parity(u - 0.5) + 0.5
    p = np.where((L.sqdist(u - b) < L.sqdist(u - a))[:, None], b, a)
    assert not np.array_equal(L.sqdist(u - p), best)
    assert not np.array_equal(L.sqdist(u - L.d_round(u)), best)
