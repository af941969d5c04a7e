"""Pins for the oracle's Rice coder, strip, scale rule and encode/decode (CPU)."""

import itertools
import math

import numpy as np
import pytest
import torch

from oracle import codec, hadamard, lattices as L, rice, splitmix
import workloads

G = {"E8": 929 / 12960, "D4": 13 / (120 * math.sqrt(2)), "A2": 5 / (36 * math.sqrt(3)), "Z": 1 / 12}


# ------------------------------------------------------------------- Rice

def test_zigzag_values_and_bijection():
    z = np.arange(-128, 128)
    q = rice.zigzag(z)
    assert list(rice.zigzag([0, -1, 1, -2, 2, 127, -128])) == [0, 1, 2, 3, 4, 254, 255]
    assert sorted(q) == list(range(256))
    assert np.array_equal(rice.unzigzag(q), z)


def _explicit_code(zeta, k):
    """The code as a string: unary quotient, terminating zero, k LSB-first bits."""
    return "1" * (zeta >> k) + "0" + "".join(str((zeta >> b) & 1) for b in range(k))


def test_code_length_closed_form():
    for zeta in range(0, 300, 7):
        for k in range(0, 16):
            assert rice.code_length(zeta, k) == len(_explicit_code(zeta, k))


def test_best_k_is_optimal_by_exhaustion():
    rng = np.random.default_rng(0)
    for scale in (0.3, 1.0, 3.0, 10.0, 40.0):
        idx = np.clip(np.rint(rng.laplace(0, scale, size=(50, 256))), -128, 127).astype(int)
        k, pay = rice.best_k(idx)
        for t in range(len(idx)):
            lens = [sum(len(_explicit_code(int(q), kk)) for q in rice.zigzag(idx[t]))
                    for kk in range(16)]
            assert pay[t] == min(lens) and k[t] == lens.index(min(lens))


def test_pack_unpack_roundtrip_and_bit_counts():
    rng = np.random.default_rng(1)
    idx = np.clip(np.rint(rng.normal(0, 4, size=(40, 256))), -128, 127).astype(int)
    idx[3] = 0                                   # all-zero tile
    idx[4] = 127                                 # extreme tile
    idx[5, ::2] = -128
    cw = rng.integers(0, 2**32, size=(40, 1), dtype=np.uint64).astype(np.uint32)
    k, tb, words, off = rice.pack(idx, cw, 32)
    assert np.array_equal(np.diff(off), (tb + 31) // 32)
    back, cbits, kk = rice.unpack(words, off, 256, 32)
    assert np.array_equal(back, idx) and np.array_equal(kk, k)
    assert np.array_equal(cbits, rice.coset_bit_rows(cw, 32))
    # the first tile's stream, bit by bit, against the explicit codes
    bits = np.unpackbits(words[off[0]:off[1]].view(np.uint8), bitorder="little")
    head = "".join(str((int(k[0]) >> b) & 1) for b in range(4))
    head += "".join(str(b) for b in rice.coset_bit_rows(cw[:1], 32)[0])
    body = "".join(_explicit_code(int(q), int(k[0])) for q in rice.zigzag(idx[0]))
    s = head + body
    assert "".join(map(str, bits[:len(s)])) == s and not bits[len(s):].any()


def test_rice_payload_close_to_index_entropy():
    """The pages put Rice within about 0.1 bps of the lattice's RD ideal; here
    the payload is compared with the empirical per-index entropy."""
    x = workloads.small_fp32()
    e = codec.encode(x, "E8", 256, 4.0, rht_seed=1)
    _, counts = np.unique(e["idx"], return_counts=True)
    p = counts / counts.sum()
    H = -(p * np.log2(p)).sum()
    pay = codec.itemized_rate(e["tile_bits"], "E8", 256)["bps_payload"]
    assert 0.0 <= pay - H < 0.15


# ------------------------------------------------------------------ strip

def test_strip_unstrip_bijection_exhaustive_small():
    vals = range(-3, 4)
    z8 = np.array([v for v in itertools.product(vals, repeat=8) if sum(v) % 2 == 0][::7])
    for c in (0, 1):
        cc = np.full((len(z8), 1), c)
        s = codec.strip(z8[None], cc[None], "E8")
        assert np.array_equal(codec.unstrip(s, "E8")[0], z8)
    z4 = np.array([v for v in itertools.product(range(-6, 7), repeat=4) if sum(v) % 2 == 0])
    s = codec.strip(z4[None], np.zeros((1, len(z4)), int), "D4")
    assert np.array_equal(codec.unstrip(s, "D4")[0], z4)


def test_strip_saves_the_membership_bits():
    # the stored last coordinate is half the true one (one bit dropped)
    z = np.array([[[1, 2, 3, 4, 5, 6, 7, 8]]])
    s = codec.strip(z, np.zeros((1, 1), int), "E8")
    assert list(s[0]) == [1, 2, 3, 4, 5, 6, 7, 4]
    z = np.array([[[0, 0, 0, 0, 0, 0, 1, -3]]])
    assert codec.strip(z, np.zeros((1, 1), int), "E8")[0, 7] == -2


# ------------------------------------------------------------ scale rule

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-3, 20000),
                        np.ldexp(1 + np.arange(512) / 512.0, 3)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(codec.bf16_rne(v.astype(np.float64)), ref)
    # fp64 inputs round directly (no double rounding through fp32)
    x = 1.0 + 2.0**-8 + 2.0**-40            # just above a bf16 midpoint
    assert codec.bf16_rne(np.array([x]))[0] == 1.0 + 2.0**-7


def test_scale_constants_closed_form():
    c = codec.scale_constant
    assert math.isclose(c("E8", 4), math.sqrt(2 * math.pi * math.e) / 16, rel_tol=1e-15)
    assert math.isclose(c("E8", 4), 0.2582955, rel_tol=1e-6)
    assert math.isclose(c("D4", 0) ** 4 * 2, (2 * math.pi * math.e) ** 2, rel_tol=1e-12)
    assert math.isclose(c("A2", 0) ** 2 * math.sqrt(3) / 2, 2 * math.pi * math.e, rel_tol=1e-12)
    assert codec.index_range_ok("E8", 256, 5) and not codec.index_range_ok("E8", 256, 6)


@pytest.mark.parametrize("lat,n", [("E8", 256), ("D4", 128), ("A2", 128), ("Z", 128)])
@pytest.mark.parametrize("bps", [4.0, 5.0])
def test_high_rate_mse_prediction(lat, n, bps):
    """MSE / sigma^2 approaches 2 pi e G 2^-2R at high rate (Gaussian input)."""
    x = np.random.default_rng(2).standard_normal((256, 1024))
    e = codec.encode(x, lat, n, bps, rht_seed=1)
    xh = codec.decode(e["idx"], e["coset"], e["scale"], lat, n, rht_seed=1)
    ratio = np.mean((xh - codec.tiles(x, n)) ** 2) / (2 * math.pi * math.e * G[lat] * 2 ** (-2 * bps))
    assert 0.95 < ratio < 1.05, ratio


def test_auto_scale_rule_and_zero_tile():
    x = np.zeros((2, 256)); x[1] = np.linspace(-1, 1, 256)
    d = codec.auto_scale(x, "E8", 4.0)
    assert d[0] == 1.0
    rms = math.sqrt(np.mean(x[1] ** 2))
    assert d[1] == codec.bf16_rne(np.array([rms * codec.scale_constant("E8", 4.0)]))[0]
    e = codec.encode(x, "E8", 256, 4.0, rht_seed=0)
    assert not e["idx"][0].any() and not e["coset"][0].any()


# --------------------------------------------------------- encode / decode

def test_quantizer_input_grid_and_formula():
    x = workloads.bf16_bits_to_f64(workloads.llama_matrix(1, shape=(8, 4096)))
    e = codec.encode(x, "E8", 256, 4.0, rht_seed=0)
    U = e["u"] * codec.GRID
    assert np.array_equal(U, np.rint(U))
    # the grid value is within half a step of the real y / Delta
    y = hadamard.forward(codec.tiles(x, 256), splitmix.rht_signs(0, 256))
    assert np.max(np.abs(e["u"] - y / e["scale"][:, None])) <= 0.5 / codec.GRID * (1 + 1e-9)


def _rne_exact(a, b):
    """rne of the exact rational product (the definition, with Fractions)."""
    from fractions import Fraction
    q = Fraction(float(a)) * Fraction(float(b))
    f = math.floor(q)
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return float(f)


def test_grid_rounds_the_exact_product_once():
    # Reading R3: U = rne(S K) of the exact product.  Checked against the
    # rational definition on pipeline-sized values and on products whose
    # fp64 rounding lands exactly on a half-integer while the exact product
    # does not (there rounding twice, rint(RN(S K)), picks the even neighbour
    # regardless of the side the product lies on).
    rng = np.random.default_rng(31)
    a = rng.normal(0.0, 3.0, 4000) * 2.0 ** rng.integers(-8, 8, 4000)
    b = rng.uniform(1.0, 2.0, 4000) * 2.0 ** 24
    got = codec.rne_product(a, b)
    assert all(g == _rne_exact(x, y) for g, x, y in zip(got, a, b))
    from fractions import Fraction
    hard = []
    for m in rng.integers(2 ** 20, 2 ** 30, 20000):
        for k in (3.0, 5.0, 7.0, 11.0):
            x = k
            y = (float(m) + 0.5) / k
            if x * y == float(m) + 0.5 and Fraction(x) * Fraction(y) != Fraction(2 * int(m) + 1, 2):
                hard.append((x, y))
        if len(hard) >= 40:
            break
    assert len(hard) >= 20
    xs = np.array([h[0] for h in hard])
    ys = np.array([h[1] for h in hard])
    got = codec.rne_product(xs, ys)
    want = np.array([_rne_exact(x, y) for x, y in hard])
    assert np.array_equal(got, want)
    # ...where rounding twice would have differed on some of them
    assert np.any(np.rint(xs * ys) != want)


@pytest.mark.parametrize("lat,n", [("E8", 256), ("E8", 128), ("D4", 128), ("A2", 128), ("Z", 128)])
def test_roundtrip_error_within_covering_radius(lat, n):
    x = workloads.bf16_bits_to_f64(workloads.llama_matrix(0, shape=(16, 4096)))
    e = codec.encode(x, lat, n, 4.0, rht_seed=3)
    X = codec.tiles(x, n)
    s = splitmix.rht_signs(3, n)
    y = hadamard.forward(X, s)
    yh = hadamard.forward(codec.decode(e["idx"], e["coset"], e["scale"], lat, n, rht_seed=3), s)
    d = codec.DIM[lat]
    err = ((y - yh) / e["scale"][:, None]).reshape(len(X), -1, d)
    if lat == "A2":
        err[..., 1] /= math.sqrt(3)
        rad2 = L.sqdist(err, L.A2_METRIC)
        cov = 1 / 3                     # (1/sqrt3)^2
    else:
        rad2 = L.sqdist(err)
        cov = {"E8": 1.0, "D4": 1.0, "Z": 0.25}[lat]
    assert rad2.max() <= cov + 1e-6


@pytest.mark.parametrize("lat,n", [("E8", 256), ("D4", 128), ("A2", 128), ("Z", 128)])
def test_reencoding_a_decoded_tile_is_idempotent(lat, n):
    x = np.random.default_rng(6).standard_normal((8, 1024))
    e = codec.encode(x, lat, n, 4.0, rht_seed=2)
    xh = codec.decode(e["idx"], e["coset"], e["scale"], lat, n, rht_seed=2)
    e2 = codec.encode(xh, lat, n, 4.0, rht_seed=2, scale=e["scale"])
    assert np.array_equal(e2["idx"], e["idx"]) and np.array_equal(e2["coset"], e["coset"])


def test_e8_decode_exact_in_fp32():
    """For n = 256 the decoded value Delta (H P) / 32 has at most 21
    significant bits, so rounding to fp32 loses nothing."""
    x = workloads.bf16_bits_to_f64(workloads.llama_matrix(2, shape=(8, 4096)))
    e = codec.encode(x, "E8", 256, 5.0, rht_seed=0)
    xh = codec.decode(e["idx"], e["coset"], e["scale"], "E8", 256, rht_seed=0)
    assert np.array_equal(xh.astype(np.float32).astype(np.float64), xh)


def test_itemized_rate_items_on_a_hand_computed_case():
    """Two E8/256 tiles worked by hand.  Tile 0 stores 256 zeros: zeta = 0,
    L(k) = 256 (1 + k), so k = 0 and the payload is 256 bits; tile_bits =
    4 + 32 + 256 = 292, 10 words, 28 padding bits.  Tile 1 stores 256 ones:
    zeta = 2, L(0) = L(1) = L(2) = 768, the smallest k (0) is taken; tile_bits
    = 4 + 32 + 768 = 804, 26 words, 28 padding bits."""
    idx = np.zeros((2, 256), np.int64)
    idx[1] = 1
    k, tb = rice.tile_bits(idx, codec.coset_bits_per_tile("E8", 256))
    assert k.tolist() == [0, 0] and tb.tolist() == [292, 804]
    r = codec.itemized_rate(tb, "E8", 256)
    assert r["payload"] == 256 + 768
    assert r["coset"] == 2 * 32
    assert r["k_field"] == 2 * 4
    assert r["scale"] == 2 * 16
    assert r["padding"] == 28 + 28
    assert r["offsets"] == 0
    assert r["total"] == 1024 + 64 + 8 + 32 + 56 == 1184
    assert r["bps"] == 1184 / 512 and r["bps_stream"] == 1152 / 512 and r["bps_payload"] == 2.0
    # the stream items are the packer's word count, bit for bit
    _, _, words, _ = rice.pack(idx, np.zeros((2, 1), np.uint32), 32)
    assert 32 * len(words) == r["payload"] + r["coset"] + r["k_field"] + r["padding"]
    # a store that keeps fp32 scales and a uint64 table of the 3 tile offsets
    s = codec.itemized_rate(tb, "E8", 256, scale_bits=32, offset_bits=64)
    assert s["scale"] == 64 and s["offsets"] == 3 * 64 and s["total"] == 1152 + 64 + 192


def test_itemized_rate_matches_pages_compression():
    """About 3.9x compression of bf16 weights at 4 bps ([ICLR abstract]) means
    about 4.1 bits per weight all-in; the itemized E8 rate, word padding
    included, lands there."""
    x = workloads.bf16_bits_to_f64(workloads.llama_matrix(1, shape=(256, 4096)))
    e = codec.encode(x, "E8", 256, 4.0, rht_seed=0)
    r = codec.itemized_rate(e["tile_bits"], "E8", 256)
    assert r["total"] == sum(r[k] for k in ("payload", "coset", "k_field", "scale", "padding"))
    assert 4.05 < r["bps"] < 4.45
    assert 3.6 < 16 / r["bps"] < 4.0


def test_rate_function_matches_encode():
    x = workloads.small_fp32(shape=(16, 1024))
    e = codec.encode(x, "E8", 256, 4.0, rht_seed=1)
    k, tb, total, words, off = codec.rate(e["idx"], e["coset"], "E8", 256)
    assert np.array_equal(k, e["rice_k"]) and np.array_equal(tb, e["tile_bits"])
    assert total == int(e["tile_bits"].sum()) and off[-1] == len(words)


# -------------------------------------------------------------- KV dither

def test_dither_is_uniform_on_the_voronoi_cell():
    d = codec.dither(2, 0, 20000, 128).reshape(-1, 8)
    assert np.abs(d.mean(0)).max() < 0.01
    g = np.mean(np.sum(d * d, axis=1)) / 8
    assert abs(g / G["E8"] - 1) < 0.01
    # every sample is its own nearest-point residual (inside the cell)
    z, c = L.e8_nearest(d)
    assert not z.any() and not c.any()


def test_dithered_error_is_granular_and_unbiased():
    rng = np.random.default_rng(7)
    kv = rng.standard_normal((4096, 128))
    e = codec.encode(kv, "E8", 128, 4.0, rht_seed=1, dither_seed=2)
    xh = codec.decode(e["idx"], e["coset"], e["scale"], "E8", 128, rht_seed=1, dither_seed=2)
    s = splitmix.rht_signs(1, 128)
    err = (hadamard.forward(kv, s) - hadamard.forward(xh, s)) / e["scale"][:, None]
    # E|err|^2 / 8 = G(E8) Delta^2 exactly in expectation, at any rate
    assert abs(np.mean(np.sum(err.reshape(-1, 8) ** 2, 1)) / 8 / G["E8"] - 1) < 0.01
    assert np.abs(err.mean(0)).max() < 5 * math.sqrt(G["E8"] / len(kv))


def test_dither_unbiased_per_vector_rotation_only_is_not():
    """Fix a few vectors and average the reconstruction over many dither
    seeds: the dithered average converges to the vector, the undithered
    reconstruction keeps a fixed error (unbiased only on average)."""
    rng = np.random.default_rng(12)
    kv = rng.standard_normal((4, 128))
    seeds = range(1, 401)
    acc = np.zeros_like(kv)
    for s in seeds:
        e = codec.encode(kv, "E8", 128, 2.0, rht_seed=5, dither_seed=s)
        acc += codec.decode(e["idx"], e["coset"], e["scale"], "E8", 128, rht_seed=5, dither_seed=s)
    bias_d = acc / len(seeds) - kv
    e0 = codec.encode(kv, "E8", 128, 2.0, rht_seed=5)
    bias_0 = codec.decode(e0["idx"], e0["coset"], e0["scale"], "E8", 128, rht_seed=5) - kv
    sd = e0["scale"][:, None] * math.sqrt(G["E8"]) / math.sqrt(len(seeds))
    assert np.sqrt(np.mean((bias_d / sd) ** 2)) < 1.3          # pure noise
    assert np.sqrt(np.mean(bias_0 ** 2)) > 3 * np.sqrt(np.mean(bias_d ** 2))
