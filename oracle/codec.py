"""Encode / decode pipeline (oracle side; test infrastructure).

Stage order from [arXiv abstract] items (i)-(iv) and [ICLR abstract]:
per-tile randomized Hadamard rotation -> nearest lattice point -> lossless
strip -> Rice rate; decoding runs the algebra backwards (index -> lattice point
-> inverse rotation), and the KV variant adds a subtractive dither.

Readings taken where the pages are silent (all stated once here):

R1 Tile: n consecutive elements of the row-major matrix (flat elements
   [n t, n t + n)); the column count must be a multiple of n.
R2 Scale, auto mode: Delta_t = bf16_rne(rms_t * c(L, R)) with
   rms_t = sqrt(sum x^2 / n) and the high-resolution constant
   c(L, R) = sqrt(2 pi e) 2^-R / vol(L)^(1/d), so that the index entropy is
   about R bits per scalar; Delta_t = 1 for a tile whose scale rounds to zero
   (an all-zero tile).  bf16 rounding makes the 16-bit scale field lossless.
R3 Quantizer input: u = y / Delta with y = H (s x) / sqrt(n), formed as
   S * K_t where S = H (s x) (exact) and K_t = 2^24 / (sqrt(n) * Delta_t)
   (two fp64 roundings: the product sqrt(n)*Delta_t, then the quotient), and
   held on a 2^-24 grid: U = rne(S * K_t), the exact product rounded once to
   the nearest integer (ties to even), u = U 2^-24.  On this grid every
   nearest-point decision, distance and margin is exact in fp64, so any two
   correct implementations agree bit for bit, ties included.  (For A2 the
   second coordinate of each pair is taken as u2/sqrt3 with
   K3_t = 2^24 / ((sqrt(n) * Delta_t) * sqrt(3)).)
R4 Strip (lossless): E8 stores (c, z0..z6, floor(z7/2)) with z = p - c/2 in
   D8 and c the coset bit; D4 stores (z0, z1, z2, floor(z3/2)); A2 stores
   (c, a, b) for the point (a + c/2, sqrt3 (b + c/2)); Z stores z.  The
   dropped bit is the parity fixed by the even coordinate sum.  Indices are
   int8; coset bits are packed LSB-first, block j at bit j, into uint32 words
   per tile.
R5 Decode: x = s * ((H (Delta p)) * (1/sqrt(n))); output fp32 by rounding the
   fp64 value, bf16 by rounding it to nearest even.
R6 KV dither (E8 only): per vector v, w = the dither box sample, d = w - Q(w)
   per 8-block (uniform over the Voronoi cell); encode Q(u + d); decode
   Delta (p - d).
R7 Per-tile rate control (a variant the pages list as a direction only):
   instead of the fixed constant, each tile's scale is searched over bf16
   values so that the tile fits a budget of floor(R n) bits (k field, coset
   bits and Rice payload; the 16-bit scale is itemized apart).  A scale is
   feasible when its indices fit int8 and tile_bits <= the budget.  The
   search runs over the bf16 bit patterns (ordered like the values) from
   the automatic scale's pattern a: lo = max(a - 1024, 0x0080),
   hi = min(a + 1024, 0x7F7F) (eight binades each way, normal values only).
   If hi is infeasible the tile takes hi; otherwise bisection with
   mid = floor((lo + hi) / 2), keeping hi feasible, until hi - lo = 1, and
   the tile takes hi.  All-zero and non-finite tiles keep the automatic
   scale.
"""

import math

import numpy as np

from . import hadamard, lattices, rice, splitmix

LATTICES = ("E8", "D4", "A2", "Z")
DIM = {"E8": 8, "D4": 4, "A2": 2, "Z": 1}
GRID = 2.0 ** 24
INT8_MIN, INT8_MAX = -128, 127


def vol_root(lattice):
    """vol(L)^(1/d) for the textbook normalisations (E8, Z: 1; D4: vol 2;
    A2 with minimum distance 1: vol sqrt3/2)."""
    if lattice in ("E8", "Z"):
        return 1.0
    if lattice == "D4":
        return math.sqrt(math.sqrt(2.0))
    if lattice == "A2":
        return math.sqrt(math.sqrt(3.0) / 2.0)
    raise ValueError(lattice)


def scale_constant(lattice, bps):
    """c(L, R) = sqrt(2 pi e) 2^-R / vol^(1/d)   (reading R2)."""
    return math.sqrt(2.0 * math.pi * math.e) * (2.0 ** (-bps)) / vol_root(lattice)


def coset_bits_per_tile(lattice, n):
    return {"E8": n // 8, "A2": n // 2, "D4": 0, "Z": 0}[lattice]


def coset_words_per_tile(lattice, n):
    return (coset_bits_per_tile(lattice, n) + 31) // 32


def index_range_ok(lattice, n, bps):
    """Auto-scale range bound: |index| <= sqrt(n)/c + 2 must fit int8."""
    return math.sqrt(n) / scale_constant(lattice, bps) + 2.0 <= INT8_MAX


# ------------------------------------------------------------- bf16 helpers

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
BF16_MIN_NORMAL = 2.0 ** -126


def bf16_rne(v):
    """Round fp64 values to the nearest bf16 value (ties to even), as fp64.

    Magnitudes below the smallest normal bf16 flush to zero (not reached by
    any scale of a nonzero tile of normal inputs); overflow gives inf.
    """
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)
    r = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    r = np.where(np.abs(r) < BF16_MIN_NORMAL, 0.0 * v, r)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, v), r)


def bf16_bits(v):
    """uint16 bit patterns of fp64 values that are exactly bf16."""
    f = np.asarray(v, np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(b):
    b = np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------- stages

def tiles(x, n):
    """Reading R1: the row-major matrix viewed as (n_tiles, n) float64."""
    x = np.asarray(x)
    if x.ndim == 2 and x.shape[1] % n:
        raise ValueError("column count must be a multiple of the tile size")
    return np.asarray(x, np.float64).reshape(-1, n)


def auto_scale(X, lattice, bps):
    """Reading R2 (per-tile RMS times the fixed constant, bf16-rounded)."""
    n = X.shape[1]
    rms = np.sqrt(np.sum(X * X, axis=1) / n)
    d = bf16_rne(rms * scale_constant(lattice, bps))
    return np.where(d == 0.0, 1.0, d)


def _split(x):
    """Veltkamp's split of float64 x into hi + lo, each of <= 26 significant
    bits, so that products of the halves are exact."""
    c = 134217729.0 * x            # 2^27 + 1
    hi = c - (c - x)
    return hi, x - hi


def rne_product(a, b):
    """rne(a b) of the exact product of float64 arrays (one rounding to the
    nearest integer, ties to even), as float64.  p = RN(a b) and the error
    e = a b - p are found exactly (Dekker's product, 1971); rint(p) is the
    answer unless p is a half-integer, where the sign of e decides."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    p = a * b
    ah, al = _split(a)
    bh, bl = _split(b)
    e = ((ah * bh - p) + ah * bl + al * bh) + al * bl
    r = np.rint(p)
    half = np.abs(p - r) == 0.5
    r = np.where(half & (e > 0), np.floor(p) + 1.0, r)
    r = np.where(half & (e < 0), np.floor(p), r)
    return r


def quantizer_input(S, delta, lattice):
    """Reading R3: U = rne(S K_t) of the exact product on the 2^-24 grid;
    returns u = U 2^-24 (for A2, odd coordinates hold u2/sqrt3)."""
    n = S.shape[1]
    t = math.sqrt(n) * np.asarray(delta, np.float64)
    K = GRID / t
    Kc = np.repeat(K[:, None], n, axis=1)
    if lattice == "A2":
        Kc[:, 1::2] = (GRID / (t * math.sqrt(3.0)))[:, None]
    return rne_product(S, Kc) / GRID


def nearest(u, lattice):
    """Nearest lattice point per block.  Returns (ints, cosets, point_w) where
    point_w is the point in decision coordinates, shape like u."""
    T, n = u.shape
    d = DIM[lattice]
    ub = u.reshape(T, n // d, d)
    if lattice == "E8":
        z, c = lattices.e8_nearest(ub)
        return z, c, lattices.e8_point(z, c).reshape(T, n)
    if lattice == "D4":
        z = lattices.d4_nearest(ub)
        return z, np.zeros(z.shape[:2], np.int64), z.astype(np.float64).reshape(T, n)
    if lattice == "A2":
        ab, c = lattices.a2_nearest(ub)
        return ab, c, (ab + 0.5 * c[..., None]).reshape(T, n)
    z = lattices.z_nearest(ub)
    return z, np.zeros(z.shape[:2], np.int64), z.astype(np.float64).reshape(T, n)


def margins(u, point_w, lattice):
    """Near-tie margin per block (0 on an exact tie), in lattice units."""
    T, n = u.shape
    d = DIM[lattice]
    x = (u - point_w).reshape(T, n // d, d)
    roots = {"E8": lattices.E8_ROOTS, "D4": lattices.D4_ROOTS,
             "A2": lattices.A2_ROOTS, "Z": lattices.Z_ROOTS}[lattice]
    metric = lattices.A2_METRIC if lattice == "A2" else None
    return lattices.margin(x, roots, metric)


def strip(z, c, lattice):
    """Reading R4: block integers -> stored indices (int64 (T, n))."""
    T = z.shape[0]
    s = np.array(z, np.int64, copy=True)
    if lattice == "E8":
        s[..., 7] = np.floor_divide(s[..., 7], 2)
    elif lattice == "D4":
        s[..., 3] = np.floor_divide(s[..., 3], 2)
    return s.reshape(T, -1)


def unstrip(idx, lattice):
    """Inverse of strip: stored indices -> block integers (T, blocks, d)."""
    idx = np.asarray(idx, np.int64)
    T = idx.shape[0]
    d = DIM[lattice]
    z = idx.reshape(T, -1, d).copy()
    if lattice == "E8":
        z[..., 7] = 2 * z[..., 7] + np.mod(np.sum(z[..., :7], axis=-1), 2)
    elif lattice == "D4":
        z[..., 3] = 2 * z[..., 3] + np.mod(np.sum(z[..., :3], axis=-1), 2)
    return z


def pack_cosets(c, lattice, n):
    """Coset bits (T, blocks) -> uint32 words (T, words), block j at bit j."""
    T = c.shape[0]
    nb = coset_bits_per_tile(lattice, n)
    nw = coset_words_per_tile(lattice, n)
    out = np.zeros((T, nw), np.uint32)
    for j in range(nb):
        out[:, j // 32] |= (c[:, j].astype(np.uint32) << np.uint32(j % 32))
    return out


def unpack_cosets(words, lattice, n):
    nb = coset_bits_per_tile(lattice, n)
    T = len(words)
    if nb == 0:
        return np.zeros((T, n // DIM[lattice]), np.int64)
    return rice.coset_bit_rows(np.asarray(words).reshape(T, -1), nb).astype(np.int64)


def full_coords(z, c, lattice):
    """Integer coordinates of the point: E8 2p; A2 2 * (point in w); D4, Z p."""
    T = z.shape[0]
    if lattice in ("E8", "A2"):
        return (2 * z + c[..., None]).reshape(T, -1)
    return z.reshape(T, -1)


def dither(dither_seed, dither_base, n_vectors, n):
    """Reading R6: d = w - Q_E8(w) per 8-block, float64 (V, n)."""
    v = np.arange(n_vectors, dtype=np.uint64) + np.uint64(dither_base)
    w = splitmix.dither_box(dither_seed, v, n)
    z, c = lattices.e8_nearest(w.reshape(n_vectors, n // 8, 8))
    return w - lattices.e8_point(z, c).reshape(n_vectors, n)


# ------------------------------------------------------------------ encode

RC_SPAN = 1024        # bf16 patterns searched on each side of the automatic scale
BF16_LOWEST_NORMAL_BITS, BF16_HIGHEST_BITS = 0x0080, 0x7F7F


def rate_controlled_scale(X, S, lattice, bps):
    """Reading R7: per-tile scales by bisection on bf16 patterns so that each
    tile fits floor(R n) bits.  X: the tiles (T, n); S = H (s x), unnormalized."""
    T, n = X.shape
    base = auto_scale(X, lattice, bps)
    budget = math.floor(bps * n)
    cb = coset_bits_per_tile(lattice, n)
    active = np.all(np.isfinite(X), axis=1) & (np.sum(X * X, axis=1) > 0.0)
    a = bf16_bits(np.where(active, base, 1.0)).astype(np.int64)
    lo = np.maximum(a - RC_SPAN, BF16_LOWEST_NORMAL_BITS)
    hi = np.minimum(a + RC_SPAN, BF16_HIGHEST_BITS)
    Sa = np.where(active[:, None], S, 0.0)   # inactive tiles: results unused

    def feasible(codes):
        delta = bf16_from_bits(codes.astype(np.uint16))
        u = quantizer_input(Sa, delta, lattice)
        z, c, _ = nearest(u, lattice)
        idx = strip(z, c, lattice)
        fits = ~np.any((idx < INT8_MIN) | (idx > INT8_MAX), axis=1)
        _, tb = rice.tile_bits(np.clip(idx, INT8_MIN, INT8_MAX), cb)
        return fits & (tb <= budget)

    run = active & feasible(hi)
    while True:
        run = run & (hi - lo > 1)
        if not run.any():
            break
        mid = (lo + hi) // 2
        f = feasible(mid)
        hi = np.where(run & f, mid, hi)
        lo = np.where(run & ~f, mid, lo)
    return np.where(active, bf16_from_bits(hi.astype(np.uint16)), base)


def encode(x, lattice="E8", n=256, bps=4.0, rht_seed=0, scale=None,
           dither_seed=None, dither_base=0, rate_control=False):
    """Encode a row-major matrix (or (V, n) KV vectors) tile by tile.

    scale: None for auto mode (reading R2) or explicit per-tile Delta values.
    dither_seed: None, or the KV dither seed (E8 only, reading R6).
    rate_control: per-tile scales by reading R7 (scale must be None; no dither).
    Returns a dict of numpy arrays: scale (float64), idx (int64 (T, n)),
    coset (uint32 (T, words)), rice_k, tile_bits, coords, margin
    (T, blocks), overflow (bool (T,)), u (the quantizer input), S.
    """
    if lattice not in LATTICES:
        raise ValueError(lattice)
    X = tiles(x, n)
    T = X.shape[0]
    signs = splitmix.rht_signs(rht_seed, n)
    S = hadamard.unnormalized_forward(X, signs)
    if rate_control:
        if scale is not None or dither_seed is not None:
            raise ValueError("rate control chooses the scales itself, without a dither")
        delta = rate_controlled_scale(X, S, lattice, bps)
    else:
        delta = auto_scale(X, lattice, bps) if scale is None else np.asarray(scale, np.float64)
    u = quantizer_input(S, delta, lattice)
    if dither_seed is not None:
        if lattice != "E8":
            raise ValueError("the dithered path is defined for E8 only")
        u = u + dither(dither_seed, dither_base, T, n)
    z, c, pw = nearest(u, lattice)
    idx = strip(z, c, lattice)
    overflow = np.any((idx < INT8_MIN) | (idx > INT8_MAX), axis=1)
    cw = pack_cosets(c, lattice, n)
    k, tb = rice.tile_bits(idx, coset_bits_per_tile(lattice, n))
    return {
        "scale": delta, "idx": idx, "coset": cw, "rice_k": k, "tile_bits": tb,
        "coords": full_coords(z, c, lattice), "margin": margins(u, pw, lattice),
        "overflow": overflow, "u": u, "S": S,
    }


# ------------------------------------------------------------------ decode

def lattice_points(idx, coset_words, lattice, n):
    """Stored indices + coset words -> lattice points in u space (T, n)."""
    idx = np.asarray(idx, np.int64)
    T = idx.shape[0]
    z = unstrip(idx, lattice).astype(np.float64)
    c = unpack_cosets(coset_words, lattice, n).astype(np.float64)
    if lattice == "E8":
        return (z + 0.5 * c[..., None]).reshape(T, n)
    if lattice == "A2":
        p = z + 0.5 * c[..., None]
        p[..., 1] = math.sqrt(3.0) * p[..., 1]
        return p.reshape(T, n)
    return z.reshape(T, n)


def decode(idx, coset_words, scale, lattice="E8", n=256, rht_seed=0,
           dither_seed=None, dither_base=0):
    """Reading R5 (and R6 with a dither seed): returns fp64 weights (T, n)
    before the output rounding; see to_fp32 / bf16_rne."""
    idx = np.asarray(idx, np.int64).reshape(-1, n)
    T = idx.shape[0]
    p = lattice_points(idx, coset_words, lattice, n)
    if dither_seed is not None:
        p = p - dither(dither_seed, dither_base, T, n)
    yhat = np.asarray(scale, np.float64)[:, None] * p
    signs = splitmix.rht_signs(rht_seed, n)
    return signs * ((yhat @ hadamard.sylvester(n)) * hadamard.inv_sqrt(n))


def rate(idx, coset_words, lattice, n):
    """hq_rate's result: (k, tile_bits, total bits, packed words, offsets)."""
    k, tb, words, off = rice.pack(idx, coset_words, coset_bits_per_tile(lattice, n))
    return k, tb, int(np.sum(tb)), words, off


def itemized_rate(tile_bits_arr, lattice, n, scale_bits=16, offset_bits=0):
    """Itemized rate accounting in bits ([ICLR abstract]: one itemized rate
    accounting), every item part of the total:

      payload   the Rice codes of the stored indices (tile_bits minus the k
                field and the coset bits);
      coset     one bit per E8 block (A2: per pair; D4, Z: none);
      k_field   4 bits per tile;
      scale     scale_bits per tile (16: the bf16 value of reading R2 is
                lossless in 16 bits; a store that keeps fp32 passes 32);
      padding   the zero bits that start every tile on a 32-bit word;
      offsets   offset_bits per entry of the (n_tiles + 1)-entry tile word
                offset table, for a store that keeps one (0: the stream is
                self-delimiting tile after tile).

    bps = total / weights; bps_stream counts the packed stream alone
    (payload + coset + k field + padding); bps_payload the Rice codes."""
    tb = np.asarray(tile_bits_arr, np.int64)
    T = tb.size
    cb = coset_bits_per_tile(lattice, n) * T
    kb = rice.K_FIELD_BITS * T
    payload = int(tb.sum()) - cb - kb
    pad = int((((tb + 31) // 32) * 32 - tb).sum())
    sb = scale_bits * T
    ob = offset_bits * (T + 1) if offset_bits else 0
    stream = payload + cb + kb + pad
    total = stream + sb + ob
    w = T * n
    return {"payload": payload, "coset": cb, "k_field": kb, "scale": sb, "padding": pad,
            "offsets": ob, "total": total, "bps": total / w, "bps_stream": stream / w,
            "bps_payload": payload / w}
