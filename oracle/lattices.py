"""Nearest-point rules for the four lattices (oracle side; test infrastructure).

[arXiv abstract] item (ii) and [ICLR abstract]: each rotated tile is quantized
to a low-dimensional optimal lattice, E8 by default, or D4, A2, Z.  The pages
give no decoder; the readings here are the textbook ones (Conway & Sloane,
"Fast quantizing and decoding algorithms for lattice quantizers and codes",
IEEE Trans. IT 28(2), 1982; and "Sphere Packings, Lattices and Groups", ch. 20):

* D_m = {z in Z^m : sum z even}.  D_m(v): f = rne(v) (round half to even);
  if sum f is odd, move the coordinate with the largest |v_j - f_j| (lowest
  index on ties) one step towards v_j (+1 when v_j - f_j = 0).
* E8 = D8 u (D8 + 1/2): a = D8(u), b = D8(u - 1/2) + 1/2, where the half
  coset's parity fix takes the last coordinate of largest residual (highest
  index on ties; tie rules are a free choice, and this one lets an
  implementation rank both cosets' residuals with one key per coordinate);
  keep a when |u - a|^2 <= |u - b|^2 (ties go to the integer coset), else b.
* D4: D4(u).
* A2 (minimum distance 1) = (Z x sqrt3 Z) u ((1/2, sqrt3/2) + Z x sqrt3 Z).
  Decisions are taken in w = (u1, u2/sqrt3), where A2 is Z^2 u ((1/2,1/2)+Z^2)
  under the metric diag(1, 3): round each coset coordinatewise (rne, and
  rne(w - 1/2) + 1/2), keep the closer, ties to the integer coset.
* Z: rne(u).

When the input lies on the 2^-24 grid the pipeline uses, every quantity below
(residuals, squared distances, margins) is exact in fp64, so evaluation order
does not matter.
"""

import itertools

import numpy as np


# ----------------------------------------------------------------- D_m / E8

def d_round(v, last=False):
    """Nearest point of D_m to each row of v (float64 (..., m)); float64 out.
    The parity fix goes to the first coordinate of largest residual, or to
    the last one with last=True."""
    v = np.asarray(v, np.float64)
    f = np.rint(v)
    d = v - f
    odd = (np.sum(f, axis=-1) % 2) != 0
    if last:
        m = v.shape[-1]
        j = m - 1 - np.argmax(np.abs(d)[..., ::-1], axis=-1)
    else:
        j = np.argmax(np.abs(d), axis=-1)
    dj = np.take_along_axis(d, j[..., None], axis=-1)[..., 0]
    step = np.where(dj >= 0, 1.0, -1.0)
    fix = np.zeros_like(f)
    np.put_along_axis(fix, j[..., None], (step * odd)[..., None], axis=-1)
    return f + fix


def sqdist(x, metric=None):
    """Squared norm of the rows of x under a diagonal metric (default: I)."""
    x = np.asarray(x, np.float64)
    if metric is None:
        return np.sum(x * x, axis=-1)
    return np.sum(x * x * np.asarray(metric, np.float64), axis=-1)


def e8_nearest(u):
    """Nearest E8 point to each 8-row of u.

    Returns (z, c): z int64 (..., 8) in D8, c int64 (...) in {0, 1}; the
    point is p = z + c/2.
    """
    u = np.asarray(u, np.float64)
    a = d_round(u)
    b = d_round(u - 0.5, last=True)
    da = sqdist(u - a)
    db = sqdist(u - (b + 0.5))
    pick_b = db < da
    z = np.where(pick_b[..., None], b, a)
    return z.astype(np.int64), pick_b.astype(np.int64)


def e8_point(z, c):
    return np.asarray(z, np.float64) + 0.5 * np.asarray(c, np.float64)[..., None]


def d4_nearest(u):
    """Nearest D4 point to each 4-row of u (int64 (..., 4))."""
    return d_round(u).astype(np.int64)


def z_nearest(u):
    return np.rint(np.asarray(u, np.float64)).astype(np.int64)


A2_METRIC = (1.0, 3.0)


def a2_nearest(w):
    """Nearest A2 point to each pair w = (u1, u2/sqrt3) (decision coordinates).

    Returns (ab, c): ab int64 (..., 2), c int64 (...); the point in w
    coordinates is ab + c/2, in u coordinates (a + c/2, sqrt3 (b + c/2)).
    """
    w = np.asarray(w, np.float64)
    c0 = np.rint(w)
    c1 = np.rint(w - 0.5)
    d0 = sqdist(w - c0, A2_METRIC)
    d1 = sqdist(w - (c1 + 0.5), A2_METRIC)
    pick1 = d1 < d0
    ab = np.where(pick1[..., None], c1, c0)
    return ab.astype(np.int64), pick1.astype(np.int64)


# ------------------------------------------------------- roots and margins

def _e8_roots():
    r = []
    for i, j in itertools.combinations(range(8), 2):
        for si in (1.0, -1.0):
            for sj in (1.0, -1.0):
                v = np.zeros(8)
                v[i], v[j] = si, sj
                r.append(v)
    for signs in itertools.product((0.5, -0.5), repeat=8):
        if sum(1 for s in signs if s < 0) % 2 == 0:
            r.append(np.array(signs))
    return np.array(r)


def _d4_roots():
    r = []
    for i, j in itertools.combinations(range(4), 2):
        for si in (1.0, -1.0):
            for sj in (1.0, -1.0):
                v = np.zeros(4)
                v[i], v[j] = si, sj
                r.append(v)
    return np.array(r)


E8_ROOTS = _e8_roots()          # 240 minimal (= Voronoi-relevant) vectors
D4_ROOTS = _d4_roots()          # 24
A2_ROOTS = np.array([[1.0, 0.0], [-1.0, 0.0], [0.5, 0.5], [0.5, -0.5],
                     [-0.5, 0.5], [-0.5, -0.5]])   # in w coordinates
Z_ROOTS = np.array([[1.0], [-1.0]])


def margin(x, roots, metric=None):
    """Margin mu = |x - r|^2 - |x|^2 minimised over the relevant vectors r.

    x = u - p for the chosen point p.  For a root lattice the Voronoi-relevant
    vectors are the roots, and the second-nearest lattice point to u is p + r
    for one of them, so mu is the squared-distance gap between the nearest
    and the second-nearest point (0 on an exact tie).
    """
    x = np.asarray(x, np.float64)
    m = np.ones(x.shape[-1]) if metric is None else np.asarray(metric, np.float64)
    rr = np.sum(roots * roots * m, axis=-1)             # |r|^2
    xr = (x * m) @ roots.T                               # <x, r>
    return np.min(rr - 2.0 * xr, axis=-1)


# --------------------------------------------------------------- brute force

def brute_force(u, lattice):
    """Exhaustive nearest-point search for small inputs.

    Enumerates, per coordinate, the three nearest values of each coset
    (enough: every coordinate of the nearest point lies within the covering
    radius of u).  Returns (best squared distance (...), list of candidate
    arrays, distance array (..., n_candidates)) so tests can check both the
    minimum and tie sets.
    """
    u = np.asarray(u, np.float64)
    d = u.shape[-1]
    if lattice == "E8":
        cosets, metric, member = (0.0, 0.5), None, _even_sum
    elif lattice == "D4":
        cosets, metric, member = (0.0,), None, _even_sum
    elif lattice == "A2":
        cosets, metric, member = (0.0, 0.5), A2_METRIC, None
    elif lattice == "Z":
        cosets, metric, member = (0.0,), None, None
    else:
        raise ValueError(lattice)
    offs = np.array(list(itertools.product((-1.0, 0.0, 1.0), repeat=d)))
    cands, dists = [], []
    for off in cosets:
        base = np.rint(u - off)
        cand = base[..., None, :] + offs + off            # (..., 3^d, d)
        dist = sqdist(u[..., None, :] - cand, metric)
        if member is not None:
            ok = member(cand - off)
            dist = np.where(ok, dist, np.inf)
        cands.append(cand)
        dists.append(dist)
    cand = np.concatenate(cands, axis=-2)
    dist = np.concatenate(dists, axis=-1)
    return np.min(dist, axis=-1), cand, dist


def _even_sum(z):
    return (np.sum(z, axis=-1) % 2) == 0
