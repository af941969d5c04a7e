"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every oracle input is generated here from seeds; nothing the oracle sees comes
from the GPU.  Encode parity compares the GPU's encode of x with the oracle's
encode of the same x; decode and rate parity feed the oracle's indices to
both sides.  Indices must match bit for bit except at oracle near-ties
(margin < 1e-6, at most a 1e-5 fraction); decoded values within 1e-5 * Delta
(bit-exact where the arithmetic is exact); Rice results exact.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import codec
import hq_testlib as T

pytestmark = pytest.mark.gpu

from lattice_post_quantization_amd import hq  # noqa: E402  (fails loudly if unbuilt)


def say(*a):
    print(*a, flush=True)


def midpoint_close(pre, rel=1e-9):
    """Tiles whose fp64 pre-rounding scale sits within rel of a bf16 midpoint."""
    m, e = np.frexp(np.asarray(pre, np.float64))
    t = m * 256.0
    return np.abs(t - np.floor(t) - 0.5) < rel * t


def oracle_pre_scale(X, lattice, bps):
    n = X.shape[1]
    return np.sqrt(np.sum(X * X, axis=1) / n) * codec.scale_constant(lattice, bps)


def check_encode(x_host, x_dev, lattice, n, bps, seed, tiles=None, label=""):
    """Auto-scale encode on the GPU (all tiles) vs the oracle (all or the
    sampled tiles), through both device paths: the plain call (the fast
    kernel where one exists) and a call that also exports coordinates (the
    generic kernel).  Returns the oracle result of the compared tiles."""
    X = codec.tiles(x_host, n)
    if tiles is not None:
        X = X[tiles]
    ora = codec.encode(X, lattice, n, bps, rht_seed=seed)
    skip = midpoint_close(oracle_pre_scale(X, lattice, bps))
    for coords in (False, True):
        g = hq.hq_encode_tiles(x_dev, lattice, n, bps, seed, want_coords=coords)
        torch.cuda.synchronize()
        path = "generic" if coords else "default"
        gs = T.host(g["scale"]).reshape(-1)
        gs = gs if tiles is None else gs[tiles]
        assert np.array_equal(gs.astype(np.float64)[~skip], ora["scale"][~skip]), \
            label + " scales (%s)" % path
        same = gs.astype(np.float64) == ora["scale"]
        gi = T.tile_rows(T.host(g["idx"]), n, tiles)
        gc = T.tile_rows(T.u32(g["coset"]), g["coset"].shape[1], tiles)
        keep = np.nonzero(same)[0]
        sub = {k: (v[keep] if isinstance(v, np.ndarray) and v.shape[:1] == (len(X),) else v)
               for k, v in ora.items()}
        bad, near, total, ok = T.compare_indices(gi[keep], gc[keep], sub, lattice, n,
                                                 "%s (%s)" % (label, path))
        gk = T.host(g["rice_k"]).reshape(-1)
        gb = T.u32(g["tile_bits"]).reshape(-1)
        if tiles is not None:
            gk, gb = gk[tiles], gb[tiles]
        assert np.array_equal(gk[keep][ok], sub["rice_k"][ok]), label + " rice_k (%s)" % path
        assert np.array_equal(gb[keep][ok], sub["tile_bits"][ok]), label + " bits (%s)" % path
        if coords:
            gco = T.tile_rows(T.host(g["coords"]), n, tiles)
            assert np.array_equal(gco[keep][ok], sub["coords"][ok]), label + " coords"
        say("%s [%s]: tiles %d, scale-boundary skips %d, blocks %d, mismatches %d, near-ties %d"
            % (label, path, len(X), int(skip.sum()), total, bad, near))
    return ora


def check_decode(ora, lattice, n, seed, label="", exact=True, dither_seed=None, dither_base=0,
                 wide=False):
    Tn = ora["idx"].shape[0]
    idx = torch.from_numpy(ora["idx"].astype(np.int16 if wide else np.int8)).cuda()
    cw = ora["coset"].astype(np.uint32)
    coset = torch.from_numpy(cw.view(np.int32)).cuda() if cw.size else None
    scale = torch.from_numpy(ora["scale"].astype(np.float32)).cuda()
    for out_dtype, bf in ((torch.float32, False), (torch.bfloat16, True)):
        y = hq.hq_decode_tiles(idx, coset, scale, lattice, n, seed, out_dtype,
                               dither_seed=dither_seed, dither_base=dither_base)
        torch.cuda.synchronize()
        g = (T.host(y) if not bf else codec.bf16_from_bits(T.bf16_host_bits(y))).reshape(Tn, n)
        o, raw = T.oracle_decode_like_gpu(ora["idx"], cw if cw.size else None, ora["scale"],
                                          lattice, n, seed, bf, dither_seed, dither_base)
        T.compare_decoded(g, o, raw, ora["scale"], bf, exact, "%s decode %s" % (label, out_dtype))


def check_rate(ora, lattice, n, label="", wide=False):
    idx = torch.from_numpy(ora["idx"].astype(np.int16 if wide else np.int8)).cuda()
    cw = ora["coset"].astype(np.uint32)
    coset = torch.from_numpy(cw.view(np.int32)).cuda() if cw.size else None
    r = hq.hq_rate(idx, coset, lattice, n, pack=True)
    torch.cuda.synchronize()
    k, tb, total, words, off = codec.rate(ora["idx"], cw, lattice, n)
    assert np.array_equal(T.host(r["rice_k"]).astype(np.int64), k), label + " k"
    assert np.array_equal(T.u32(r["tile_bits"]).astype(np.int64), tb), label + " bits"
    assert int(T.host(r["total_bits"])[0]) == total, label + " total"
    goff = T.host(r["tile_word_offset"])
    assert np.array_equal(goff, off), label + " offsets"
    assert np.array_equal(T.u32(r["stream"])[:off[-1]], words), label + " stream"
    # the same with the oracle's rice_k and tile_bits given (HQ_RATE_GIVEN)
    given = {"rice_k": torch.from_numpy(k.astype(np.uint8)).cuda(),
             "tile_bits": torch.from_numpy(tb.astype(np.uint32).view(np.int32)).cuda()}
    r = hq.hq_rate(idx, coset, lattice, n, pack=True, given=given)
    torch.cuda.synchronize()
    assert int(T.host(r["total_bits"])[0]) == total, label + " total (given)"
    assert np.array_equal(T.host(r["tile_word_offset"]), off), label + " offsets (given)"
    assert np.array_equal(T.u32(r["stream"])[:off[-1]], words), label + " stream (given)"


# ------------------------------------------------------------------ tests

def test_small_fp32_e8_full_parity():
    """1024x1024 fp32 N(0,1), tiles of 256, RHT seed 1, E8 at 4 bps."""
    x = workloads.small_fp32()
    say("case: small fp32 E8/256 R=4 seed 1")
    ora = check_encode(x, T.f32_device(x), "E8", 256, 4.0, 1, label="small_fp32")
    check_decode(ora, "E8", 256, 1, "small_fp32")
    check_rate(ora, "E8", 256, "small_fp32")
    # explicit oracle scales give the same indices
    g = hq.hq_encode_tiles(T.f32_device(x), "E8", 256, 4.0, 1,
                           scale=torch.from_numpy(ora["scale"].astype(np.float32)).cuda())
    torch.cuda.synchronize()
    T.compare_indices(T.host(g["idx"]).reshape(-1, 256), T.u32(g["coset"]), ora, "E8", 256,
                      "small_fp32 explicit")


@pytest.mark.parametrize("lattice,n", [(lat, n) for lat in ("E8", "D4", "A2", "Z")
                                       for n in (64, 128, 256, 512)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lattices_tile_sizes_ragged(lattice, n, dtype):
    """Every lattice x tile size on a small bf16 / fp32 matrix whose tile
    count leaves a ragged final block."""
    rows, cols = 37, 6 * n          # 222 tiles: not a multiple of 16 or 32
    rng = np.random.default_rng(21)
    w = rng.standard_normal((rows, cols)) * 0.02
    w[:, 5] *= 300.0                # an outlier column
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(w.astype(np.float32))
        xh = workloads.bf16_bits_to_f64(bits)
        xd = T.bf16_device(bits, (rows, cols))
    else:
        xh = w.astype(np.float32)
        xd = T.f32_device(xh)
    for bps in (2.0, 4.0):
        label = "%s/%d %s R=%g" % (lattice, n, dtype, bps)
        say("case:", label)
        ora = check_encode(xh, xd, lattice, n, bps, 7, label=label)
        check_decode(ora, lattice, n, 7, label, exact=(lattice != "A2"))
        check_rate(ora, lattice, n, label)


def _spike_tiles(n, seed, count):
    """Tiles whose rotation is a single spike of height sqrt(n) (x = s . H
    row i, so H(s x) = n e_i): the largest |u| the auto scale allows,
    sqrt(n) / c(L, R), reached by one coordinate."""
    from oracle import hadamard, splitmix
    s = splitmix.rht_signs(seed, n)
    H = hadamard.sylvester(n)
    rows = [s * H[(37 * i + 5) % n] * (1.0 + 0.25 * i) for i in range(count)]
    return np.asarray(rows)


@pytest.mark.parametrize("lattice,n,bps", [("E8", 256, 6.0), ("E8", 256, 7.0), ("E8", 128, 6.0),
                                           ("E8", 128, 7.0), ("D4", 128, 6.0), ("A2", 128, 7.0),
                                           ("Z", 256, 6.0), ("E8", 512, 6.0)])
def test_idx16_mode_parity(lattice, n, bps):
    """The int16 index mode (HQ_IDX16) at rates whose indices leave int8:
    a ragged bf16 matrix with an outlier column and spike tiles (one rotated
    coordinate at sqrt(n)/c), encode (both kernel paths of the generic
    encoder), decode, rate + pack and unpack against the oracle."""
    rows, cols = 37, 6 * n
    rng = np.random.default_rng(23)
    w = rng.standard_normal((rows, cols)) * 0.02
    w[:, 5] *= 300.0
    w.reshape(-1, n)[:8] = _spike_tiles(n, 9, 8) * 0.02
    bits = workloads.f32_to_bf16_bits(w.astype(np.float32))
    xh = workloads.bf16_bits_to_f64(bits)
    xd = T.bf16_device(bits, (rows, cols))
    label = "idx16 %s/%d R=%g" % (lattice, n, bps)
    say("case:", label)
    X = codec.tiles(xh, n)
    ora = codec.encode(X, lattice, n, bps, rht_seed=9)
    assert np.abs(ora["idx"]).max() > 127            # the mode is needed
    assert np.abs(ora["idx"]).max() <= 32767
    skip = midpoint_close(oracle_pre_scale(X, lattice, bps))
    for coords in (False, True):
        g = hq.hq_encode_tiles(xd, lattice, n, bps, 9, want_coords=coords, idx16=True)
        torch.cuda.synchronize()
        assert g["idx"].dtype == torch.int16
        gs = T.host(g["scale"]).astype(np.float64)
        assert np.array_equal(gs[~skip], ora["scale"][~skip]), label
        keep = np.nonzero(gs == ora["scale"])[0]
        sub = {k: (v[keep] if isinstance(v, np.ndarray) and v.shape[:1] == (len(X),) else v)
               for k, v in ora.items()}
        gi = T.host(g["idx"]).reshape(-1, n)[keep]
        gc = T.u32(g["coset"]).reshape(len(X), -1)[keep]
        bad, near, total, ok = T.compare_indices(gi, gc, sub, lattice, n, label)
        assert np.array_equal(T.host(g["rice_k"])[keep][ok], sub["rice_k"][ok]), label
        assert np.array_equal(T.u32(g["tile_bits"])[keep][ok], sub["tile_bits"][ok]), label
        if coords:
            gco = T.host(g["coords"]).reshape(-1, n)[keep]
            assert np.array_equal(gco[ok], sub["coords"][ok]), label + " coords"
        say("  %s: blocks %d, mismatches %d, near-ties %d, max |idx| %d"
            % ("coords" if coords else "plain", total, bad, near, int(np.abs(ora["idx"]).max())))
    check_decode(ora, lattice, n, 9, label, exact=(lattice != "A2"), wide=True)
    check_rate(ora, lattice, n, label, wide=True)
    # the packed stream back through the stream decoder
    idx = torch.from_numpy(ora["idx"].astype(np.int16)).cuda()
    cw = ora["coset"].astype(np.uint32)
    coset = torch.from_numpy(cw.view(np.int32)).cuda() if cw.size else None
    r = hq.hq_rate(idx, coset, lattice, n, pack=True)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    u = hq.hq_unpack(r["stream"], r["tile_word_offset"], lattice, n, status=st, idx16=True)
    torch.cuda.synchronize()
    assert int(T.host(st)[0]) == 0, label + " unpack status"
    assert np.array_equal(T.host(u["idx"]).astype(np.int64), ora["idx"]), label + " unpack idx"
    if cw.size:
        assert np.array_equal(T.u32(u["coset"]), cw), label + " unpack coset"
    assert np.array_equal(T.host(u["rice_k"]).astype(np.int64), ora["rice_k"]), label + " unpack k"


def test_idx16_caller_scale_clamp():
    """With a caller scale far below the auto one, grid values pass the
    int16 mode's clamp (|u| = 32000): the tile's status flags the overflow,
    as the oracle's indices leave int16 there."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    xd = T.f32_device(w)
    scale = torch.full((4,), 1e-7, dtype=torch.float32, device="cuda")
    scale[1:] = 1e-3
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    hq.hq_encode_tiles(xd, "E8", 256, 6.0, 1, scale=scale, status=st, idx16=True)
    torch.cuda.synchronize()
    ora = codec.encode(w.astype(np.float64), "E8", 256, 6.0, rht_seed=1,
                       scale=T.host(scale).astype(np.float64))
    big = np.abs(ora["idx"]).max(axis=1) > 32767
    assert big[0] and not big[1:].any()
    assert int(T.host(st)[0]) & hq.HQ_ST_OVERFLOW
    # the tiles inside the range match the oracle
    st.zero_()
    g = hq.hq_encode_tiles(xd[1:], "E8", 256, 6.0, 1, scale=scale[1:], status=st, idx16=True)
    torch.cuda.synchronize()
    assert int(T.host(st)[0]) == 0
    sub = {k: (v[1:] if isinstance(v, np.ndarray) and v.shape[:1] == (4,) else v)
           for k, v in ora.items()}
    T.compare_indices(T.host(g["idx"]).reshape(-1, 256), T.u32(g["coset"]), sub, "E8", 256,
                      "idx16 caller scale")


@pytest.mark.parametrize("bps", [3.0, 4.0, 5.0])
def test_llama_layer_parity(bps):
    """One Llama-3.1-8B-shaped layer in bf16 (outlier columns): k in full,
    the other six projections on every 61st tile, at 3, 4 and 5 bps."""
    for m, (name, rows, cols) in enumerate(workloads.LLAMA_LAYER):
        bits = workloads.llama_matrix(m, layer=0)
        xd = T.bf16_device(bits, (rows, cols))
        xh = workloads.bf16_bits_to_f64(bits)
        n_tiles = rows * cols // 256
        tiles = None if name == "k" else np.arange(0, n_tiles, 61)
        label = "layer0.%s R=%g" % (name, bps)
        say("case:", label)
        ora = check_encode(xh, xd, "E8", 256, bps, 0, tiles=tiles, label=label)
        if name in ("k", "down"):
            check_decode(ora, "E8", 256, 0, label)
            check_rate(ora, "E8", 256, label)
        del xd


def test_lattice_sweep_matrix():
    """The 4096x14336 bf16 sweep matrix: D4, A2, Z (tile 128) and E8 (tile
    256) at 2, 3, 4 bps; every 97th tile against the oracle; full-matrix MSE
    against the normalized-second-moment prediction."""
    bits = workloads.sweep_matrix()
    rows, cols = bits.shape
    xd = T.bf16_device(bits, (rows, cols))
    xh = workloads.bf16_bits_to_f64(bits)
    G = {"E8": 929 / 12960, "D4": 13 / (120 * math.sqrt(2)), "A2": 5 / (36 * math.sqrt(3)),
         "Z": 1 / 12}
    var = float(torch.mean(xd.double() ** 2))
    for lattice, n in (("D4", 128), ("A2", 128), ("Z", 128), ("E8", 256)):
        for bps in (2.0, 3.0, 4.0):
            label = "sweep %s/%d R=%g" % (lattice, n, bps)
            say("case:", label)
            tiles = np.arange(0, rows * cols // n, 97)
            ora = check_encode(xh, xd, lattice, n, bps, 1, tiles=tiles, label=label)
            check_decode(ora, lattice, n, 1, label, exact=(lattice != "A2"))
            g = hq.hq_encode_tiles(xd, lattice, n, bps, 1)
            y = hq.hq_decode_tiles(g["idx"], g["coset"], g["scale"], lattice, n, 1, torch.float32)
            mse = float(torch.mean((y.double() - xd.double()) ** 2)) / var
            pred = 2 * math.pi * math.e * G[lattice] * 2 ** (-2 * bps)
            say("  mse/var %.4e  prediction %.4e  ratio %.3f" % (mse, pred, mse / pred))
            assert 0.75 < mse / pred < 1.3


def test_kv_dither_parity_and_unbiasedness():
    """K and V [8, 32768, 128] bf16 with per-channel offsets; E8, 4 bps,
    subtractive dither (seed 2); every 509th vector against the oracle, a
    contiguous block through the dithered decoder, and the mean query-key
    error over 4096 queries."""
    kb, vb = workloads.kv_layer()
    nvec = kb.shape[0] * kb.shape[1]
    for name, bits, base in (("K", kb, 0), ("V", vb, nvec)):
        xd = T.bf16_device(bits, (nvec, 128))
        xh = workloads.bf16_bits_to_f64(bits).reshape(nvec, 128)
        say("case: kv", name)
        g = hq.hq_kv_encode(xd, 4.0, 1, dither_seed=2, dither_base=base)
        torch.cuda.synchronize()
        sample = np.arange(0, nvec, 509)[:300]
        # the oracle encodes each sampled vector with its own global index
        parts = [codec.encode(xh[i:i + 1], "E8", 128, 4.0, rht_seed=1, dither_seed=2,
                              dither_base=base + int(i)) for i in sample]
        ora = {k: np.concatenate([o[k] for o in parts])
               for k in ("scale", "idx", "coset", "rice_k", "tile_bits", "margin")}
        assert np.array_equal(T.host(g["scale"])[sample].astype(np.float64), ora["scale"])
        T.compare_indices(T.host(g["idx"])[sample], T.u32(g["coset"])[sample], ora, "E8", 128,
                          "kv %s" % name)
        assert np.array_equal(T.host(g["rice_k"])[sample], ora["rice_k"])
        assert np.array_equal(T.u32(g["tile_bits"])[sample], ora["tile_bits"])
        # contiguous block through both dithered decoders
        blk = slice(1000, 1512)
        ora = codec.encode(xh[blk], "E8", 128, 4.0, rht_seed=1, dither_seed=2,
                           dither_base=base + 1000)
        check_decode(ora, "E8", 128, 1, "kv %s" % name, exact=True, dither_seed=2,
                     dither_base=base + 1000)
    # unbiasedness of q . (k_hat - k)
    xd = T.bf16_device(kb, (nvec, 128))
    q = torch.from_numpy(workloads.kv_queries()).cuda()
    res = {}
    for mode, ds in (("dither", 2), ("rotation-only", None)):
        g = hq.hq_kv_encode(xd, 4.0, 1, dither_seed=ds, dither_base=0)
        y = hq.hq_decode_tiles(g["idx"], g["coset"], g["scale"], "E8", 128, 1, torch.float32,
                               dither_seed=ds, dither_base=0)
        err = (y.double() - xd.double()).reshape(8, -1, 128)
        qbar = q.mean(0)
        stat = float((err.mean(1) @ qbar).mean())            # mean over h, j, t of q_j . e
        per_tok = (err @ qbar).reshape(-1)
        se = float(per_tok.std() / math.sqrt(per_tok.numel()))
        # per-query bias z-scores b_j = q_j . mean(e) against their null spread
        e2 = err.reshape(-1, 128)
        b = q @ e2.mean(0)
        null_sd = torch.sqrt((q * q) @ (e2.var(0) / e2.shape[0]))
        z = (b / null_sd).abs()
        res[mode] = (stat, se, float(z.mean()), float(z.max()))
        say("  %s: mean q.e %.3e  SE %.3e  per-query |z| mean %.2f max %.2f" % ((mode,) + res[mode]))
    stat, se, _, _ = res["dither"]
    assert abs(stat) <= 4 * se


def test_kv_dither_unbiased_per_vector_on_the_gpu():
    """The subtractive dither makes each cached vector's reconstruction
    unbiased; rotation alone does not.  64 fixed K vectors (bf16, 4 bps,
    every 4096th vector of the K cache), each encoded and decoded (fp32) by
    the HIP path under 1024 dither seeds, and once rotation-only.  Under the
    dither the error is uniform on the E8 Voronoi cell scaled by Delta,
    independent of the vector: per coordinate mean 0 and variance
    G(E8) Delta^2, so z = mean over seeds / (Delta sqrt(G / S)) is standard
    in every coordinate of every vector, and MSE / (G Delta^2) is 1.  The
    rotation-only error is fixed per vector, of size ~ sqrt(G) Delta: its z
    grows as sqrt(S) (~32 here)."""
    g_e8 = 929.0 / 12960.0            # normalized second moment of E8 (Conway-Sloane)
    kb, _ = workloads.kv_layer()
    sel = np.arange(64) * 4096
    bits = kb.reshape(-1, 128)[sel]
    xd = T.bf16_device(bits, (64, 128))
    x = xd.double()
    n_seeds = 1024
    say("case: kv per-vector unbiasedness, 64 vectors x %d dither seeds" % n_seeds)
    o = hq.hq_kv_encode(xd, 4.0, 1, dither_seed=1)
    delta = o["scale"].double()[:, None]
    y = torch.empty((64, 128), dtype=torch.float32, device=xd.device)
    acc = torch.zeros_like(x)
    acc2 = torch.zeros_like(x)
    for s in range(1, n_seeds + 1):
        hq.hq_kv_encode(xd, 4.0, 1, dither_seed=s, out=o)
        hq.hq_decode_tiles(o["idx"], o["coset"], o["scale"], "E8", 128, 1, torch.float32,
                           dither_seed=s, out=y)
        e = y.double() - x
        acc += e
        acc2 += e * e
    assert torch.equal(o["scale"].double()[:, None], delta)    # the dither leaves the scale alone
    unit = delta * math.sqrt(g_e8 / n_seeds)
    z = acc / n_seeds / unit
    z2_vec = (z * z).mean(1)
    mse_d = float((acc2 / n_seeds / (g_e8 * delta * delta)).mean())
    o0 = hq.hq_kv_encode(xd, 4.0, 1)
    y0 = hq.hq_decode_tiles(o0["idx"], o0["coset"], o0["scale"], "E8", 128, 1, torch.float32)
    e0 = y0.double() - x
    z0 = e0 / unit
    z0_vec = torch.sqrt((z0 * z0).mean(1))
    mse_0 = float((e0 * e0 / (g_e8 * delta * delta)).mean())
    rms_z = float(torch.sqrt((z * z).mean()))
    say("  dither: rms z %.3f, max per-vector mean z^2 %.3f, MSE/(G D^2) %.4f" %
        (rms_z, float(z2_vec.max()), mse_d))
    say("  rotation-only: min per-vector rms z %.1f, MSE/(G D^2) %.4f" %
        (float(z0_vec.min()), mse_0))
    assert 0.9 < rms_z < 1.1                  # 8192 coordinates: 1 +- 0.016
    assert float(z2_vec.max()) < 1.6          # 64 vectors, chi2(128)/128: 1 +- 0.125
    assert abs(mse_d - 1.0) < 0.01
    assert float(z0_vec.min()) > 8.0          # every vector keeps a fixed error


def _attn_tol(q, k_hat, v_hat, tau):
    """Bound for hq_kv_attention against the fp64 attention of the same
    decoded cache.  A score (base-2 units, tau log2(e) q . khat) is an fp32
    sum of 128 products of fp32-rounded factors: its error is at most
    2^-16 tau log2(e) |q| max|khat| (orthonormal rotation: the rotated
    factors keep the norms).  An error ds in the scores moves the softmax
    weights by at most a factor 2^(2 ds), so the output by at most
    2 ln2 ds max|vhat|; the fp32 running sums over a range and the merge add
    at most 2^-14 max|vhat|."""
    ds = 2.0 ** -16 * tau * math.log2(math.e) * np.linalg.norm(q, axis=1) * \
        np.max(np.linalg.norm(k_hat, axis=1))
    vmax = np.max(np.abs(v_hat))
    return ((2 * math.log(2) * ds + 2.0 ** -14) * vmax)[:, None]


@pytest.mark.parametrize("dither", [True, False])
def test_kv_attention_parity(dither):
    """hq_kv_attention against the oracle's softmax attention over its own
    dithered (or rotation-only) decode of K and V: 3001 keys (ragged against
    the key ranges and the four key residues), K with RHT seed 1 and dither
    seed 2, V with RHT seed 7 and dither seed 3 at global base 3001, the K/V
    workload's distribution (N(0, 1) with per-channel offsets), 11 queries
    (three query groups), tau = 1/sqrt(128) and 0.5."""
    from oracle.attention import attention
    kb, vb = workloads.kv_layer()
    n = 3001
    kx = workloads.bf16_bits_to_f64(kb[0, :n]).reshape(n, 128)
    vx = workloads.bf16_bits_to_f64(vb[0, :n]).reshape(n, 128)
    ks = dict(rht_seed=1, dither_seed=2 if dither else None, dither_base=0)
    vs = dict(rht_seed=7, dither_seed=3 if dither else None, dither_base=n)
    say("case: kv attention n_keys=%d dither=%s" % (n, dither))
    ko = codec.encode(kx, "E8", 128, 4.0, rht_seed=1, dither_seed=ks["dither_seed"],
                      dither_base=0)
    vo = codec.encode(vx, "E8", 128, 4.0, rht_seed=7, dither_seed=vs["dither_seed"],
                      dither_base=n)
    k_hat = codec.decode(ko["idx"], ko["coset"], ko["scale"], "E8", 128, 1,
                         dither_seed=ks["dither_seed"], dither_base=0).reshape(n, 128)
    v_hat = codec.decode(vo["idx"], vo["coset"], vo["scale"], "E8", 128, 7,
                         dither_seed=vs["dither_seed"], dither_base=n).reshape(n, 128)

    def dev_enc(o):
        return {"idx": torch.from_numpy(o["idx"].astype(np.int8).reshape(n, 128)).cuda(),
                "coset": torch.from_numpy(o["coset"].astype(np.uint32).view(np.int32).reshape(n)).cuda(),
                "scale": torch.from_numpy(o["scale"].astype(np.float32)).cuda()}

    kd, vd = dev_enc(ko), dev_enc(vo)
    q = np.random.default_rng(17).standard_normal((11, 128)).astype(np.float32)
    qd = torch.from_numpy(q).cuda()
    for tau in (1.0 / math.sqrt(128.0), 0.5):
        out = hq.hq_kv_attention(qd, kd, vd, tau=tau, k_cache=ks, v_cache=vs)
        out2 = hq.hq_kv_attention(qd, kd, vd, tau=tau, k_cache=ks, v_cache=vs)
        torch.cuda.synchronize()
        ref = attention(q.astype(np.float64), k_hat, v_hat, tau)
        tol = _attn_tol(q.astype(np.float64), k_hat, v_hat, tau)
        err = np.abs(T.host(out).astype(np.float64) - ref)
        say("  tau %.4f  max err %.3e  max tol %.3e" % (tau, err.max(), tol.max()))
        assert np.all(err <= tol), "max err/tol %.3g" % np.max(err / tol)
        assert torch.equal(out, out2)


@pytest.mark.parametrize("n_keys,n_q", [(1, 5), (3, 1), (257, 8), (1029, 4)])
def test_kv_attention_small_caches(n_keys, n_q):
    """Three heads of tiny and ragged caches (fewer keys than a wave's four
    residues, one key past a range of 256) and query counts on both sides
    of the 4 / 8 query groups, against the oracle's attention over its own
    dithered decode of each head (dither index = head x n_keys + key)."""
    from oracle.attention import attention
    rng = np.random.default_rng(31 + n_keys)
    heads = 3
    x = rng.standard_normal((heads * n_keys, 128))
    xk = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(x.astype(np.float32)))
    xv = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(
        rng.standard_normal((heads * n_keys, 128)).astype(np.float32)))
    say("case: kv attention %d heads x %d keys, %d queries" % (heads, n_keys, n_q))
    ko = codec.encode(xk, "E8", 128, 4.0, rht_seed=4, dither_seed=6, dither_base=100)
    vo = codec.encode(xv, "E8", 128, 4.0, rht_seed=4, dither_seed=6, dither_base=9000)
    k_hat = codec.decode(ko["idx"], ko["coset"], ko["scale"], "E8", 128, 4, dither_seed=6,
                         dither_base=100).reshape(heads, n_keys, 128)
    v_hat = codec.decode(vo["idx"], vo["coset"], vo["scale"], "E8", 128, 4, dither_seed=6,
                         dither_base=9000).reshape(heads, n_keys, 128)
    n = heads * n_keys

    def dev_enc(o):
        return {"idx": torch.from_numpy(o["idx"].astype(np.int8).reshape(n, 128)).cuda(),
                "coset": torch.from_numpy(o["coset"].astype(np.uint32).view(np.int32).reshape(n)).cuda(),
                "scale": torch.from_numpy(o["scale"].astype(np.float32)).cuda()}

    q = rng.standard_normal((heads, n_q, 128)).astype(np.float32)
    out = hq.hq_kv_attention(torch.from_numpy(q).cuda(), dev_enc(ko), dev_enc(vo), tau=0.3,
                             k_cache=dict(rht_seed=4, dither_seed=6, dither_base=100),
                             v_cache=dict(rht_seed=4, dither_seed=6, dither_base=9000))
    torch.cuda.synchronize()
    for h in range(heads):
        ref = attention(q[h].astype(np.float64), k_hat[h], v_hat[h], 0.3)
        tol = _attn_tol(q[h].astype(np.float64), k_hat[h], v_hat[h], 0.3)
        err = np.abs(T.host(out[h]).astype(np.float64) - ref)
        assert np.all(err <= tol), "head %d: max err/tol %.3g" % (h, np.max(err / tol))


def test_kv_attention_all_heads_against_decoded_cache():
    """At the workload's size (all heads of [8, 32768, 128], dithered K and
    V encoded as one cache each, 4 queries per head in one call):
    hq_kv_attention agrees, within the same bound per head, with fp64
    attention over the same cache decoded by hq_decode_tiles (the rotated-
    domain form equals decode-then-attend), and a single key gives that
    key's decoded value."""
    kb, vb = workloads.kv_layer()
    heads, nkeys = kb.shape[0], kb.shape[1]
    say("case: kv attention %d heads x %d keys" % (heads, nkeys))
    kd = T.bf16_device(kb, (heads * nkeys, 128))
    vd = T.bf16_device(vb, (heads * nkeys, 128))
    ks = dict(rht_seed=1, dither_seed=2, dither_base=0)
    vs = dict(rht_seed=1, dither_seed=2, dither_base=heads * nkeys)
    ke = hq.hq_kv_encode(kd, 4.0, 1, dither_seed=2, dither_base=0)
    ve = hq.hq_kv_encode(vd, 4.0, 1, dither_seed=2, dither_base=heads * nkeys)
    q = torch.from_numpy(workloads.kv_queries()[:4 * heads].astype(np.float32)
                         .reshape(heads, 4, 128)).cuda()
    tau = 1.0 / math.sqrt(128.0)
    out = hq.hq_kv_attention(q, ke, ve, tau=tau, k_cache=ks, v_cache=vs)
    k_hat = hq.hq_decode_tiles(ke["idx"], ke["coset"], ke["scale"], "E8", 128, 1, torch.float32,
                               dither_seed=2, dither_base=0).double().reshape(heads, nkeys, 128)
    v_hat = hq.hq_decode_tiles(ve["idx"], ve["coset"], ve["scale"], "E8", 128, 1, torch.float32,
                               dither_seed=2, dither_base=heads * nkeys).double() \
        .reshape(heads, nkeys, 128)
    ref = torch.softmax(tau * (q.double() @ k_hat.transpose(1, 2).contiguous()), dim=2) @ v_hat
    torch.cuda.synchronize()
    for h in range(heads):
        tol = _attn_tol(T.host(q[h]).astype(np.float64), T.host(k_hat[h]), T.host(v_hat[h]), tau)
        err = np.abs(T.host(out[h]).astype(np.float64) - T.host(ref[h]))
        say("  head %d max err %.3e  max tol %.3e" % (h, err.max(), tol.max()))
        assert np.all(err <= tol), "head %d" % h
    one = {k: v[5:6] for k, v in ke.items() if k in ("idx", "coset", "scale")}
    onev = {k: v[5:6] for k, v in ve.items() if k in ("idx", "coset", "scale")}
    out1 = hq.hq_kv_attention(q[0], one, onev, tau=tau, k_cache=dict(ks, dither_base=5),
                              v_cache=dict(vs, dither_base=heads * nkeys + 5))
    torch.cuda.synchronize()
    v5 = T.host(v_hat[0, 5]).astype(np.float64)
    assert np.all(np.abs(T.host(out1).astype(np.float64) - v5[None, :]) <= 2.0 ** -20 * np.abs(v5).max())


def test_edge_cases_and_status_bits():
    dev = torch.device("cuda")
    # empty input: no-op
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    g = hq.hq_encode_tiles(x, "E8", 256, 4.0, 0)
    assert g["idx"].numel() == 0
    # zero tiles -> scale 1, zero indices; a single tile; odd shapes
    x = torch.zeros((1, 512), dtype=torch.bfloat16, device=dev)
    g = hq.hq_encode_tiles(x, "E8", 256, 4.0, 0)
    torch.cuda.synchronize()
    assert np.all(T.host(g["scale"]) == 1.0) and not T.host(g["idx"]).any()
    # non-finite input sets the status bit
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    x = torch.randn((2, 256), device=dev).to(torch.bfloat16)
    x[1, 17] = float("nan")
    hq.hq_encode_tiles(x, "E8", 256, 4.0, 0, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & hq.HQ_ST_NONFINITE
    # tile 512 (two halves of 256 on neighbouring lanes): zero tiles, and a
    # non-finite element in either half flags the call and leaves the
    # finite tiles beside it as they were
    x = torch.zeros((3, 512), dtype=torch.bfloat16, device=dev)
    g = hq.hq_encode_tiles(x, "E8", 512, 4.0, 0)
    torch.cuda.synchronize()
    assert np.all(T.host(g["scale"]) == 1.0) and not T.host(g["idx"]).any()
    for col in (17, 300):
        st.zero_()
        x = torch.randn((3, 512), device=dev).to(torch.bfloat16)
        ref = hq.hq_encode_tiles(x, "E8", 512, 4.0, 0)
        x[1, col] = float("nan")
        g = hq.hq_encode_tiles(x, "E8", 512, 4.0, 0, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) & hq.HQ_ST_NONFINITE, col
        for k in ("scale", "rice_k", "tile_bits"):
            assert torch.equal(g[k][[0, 2]], ref[k][[0, 2]]), (col, k)
        assert torch.equal(g["idx"].reshape(3, 512)[[0, 2]], ref["idx"].reshape(3, 512)[[0, 2]])
    st.zero_()
    # an explicit scale far too small overflows the int8 indices
    st.zero_()
    x = torch.randn((1, 256), device=dev).to(torch.bfloat16)
    hq.hq_encode_tiles(x, "E8", 256, 4.0, 0, scale=torch.full((1,), 1e-4, device=dev),
                       status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & hq.HQ_ST_OVERFLOW
    # a packed stream with too little capacity
    st.zero_()
    x = torch.randn((4, 1024), device=dev).to(torch.bfloat16)
    g = hq.hq_encode_tiles(x, "E8", 256, 4.0, 0)
    r = hq.hq_rate(g["idx"], g["coset"], "E8", 256, pack=True, capacity_words=40, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & hq.HQ_ST_STREAM_FULL
    # auto scale outside the int8 range is refused before launch
    with pytest.raises(hq.HQError) as e:
        hq.hq_encode_tiles(x, "E8", 256, 6.0, 0)
    assert e.value.code == hq.HQ_ERANGE


def test_bitwise_determinism():
    bits = workloads.llama_matrix(1, layer=3)
    xd = T.bf16_device(bits, bits.shape)
    a = hq.hq_encode_tiles(xd, "E8", 256, 4.0, 3)
    b = hq.hq_encode_tiles(xd, "E8", 256, 4.0, 3)
    ya = hq.hq_decode_tiles(a["idx"], a["coset"], a["scale"], "E8", 256, 3)
    yb = hq.hq_decode_tiles(b["idx"], b["coset"], b["scale"], "E8", 256, 3)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))


@pytest.mark.parametrize("n", [256, 512])
def test_batched_calls_match_single_calls_and_oracle(n):
    """hq_encode_batch / hq_decode_batch over mixed matrix sizes (more than
    eight, one empty, ragged tile counts) give the same bytes as one call per
    matrix, and sampled tiles match the oracle (E8, tiles of 256 and 512)."""
    rng = np.random.default_rng(31)
    shapes = [(r, c * n // 256) for r, c in
              [(7, 256), (1, 512), (0, 256), (33, 768), (16, 256), (5, 1024), (40, 256),
               (3, 256), (9, 512), (2, 2048), (64, 256)]]
    mats, hosts = [], []
    for r, c in shapes:
        w = rng.standard_normal((r, c)) * 0.02
        bits = workloads.f32_to_bf16_bits(w.astype(np.float32))
        hosts.append(workloads.bf16_bits_to_f64(bits))
        mats.append(T.bf16_device(bits, (r, c)))
    say("case: batch of %d matrices" % len(mats))
    for bps in (3.0, 4.0):
        batch = hq.hq_encode_batch(mats, "E8", n, bps, 9)
        ys = hq.hq_decode_batch(batch, "E8", n, 9, torch.bfloat16)
        torch.cuda.synchronize()
        for i, (x, b, y) in enumerate(zip(mats, batch, ys)):
            if x.numel() == 0:
                continue
            s = hq.hq_encode_tiles(x, "E8", n, bps, 9)
            ys1 = hq.hq_decode_tiles(s["idx"], s["coset"], s["scale"], "E8", n, 9)
            torch.cuda.synchronize()
            for k in ("scale", "idx", "coset", "rice_k", "tile_bits"):
                assert torch.equal(b[k], s[k]), (i, k)
            assert torch.equal(y.view(torch.int16), ys1.view(torch.int16)), i
            ora = codec.encode(hosts[i], "E8", n, bps, rht_seed=9)
            assert np.array_equal(T.host(b["scale"]).astype(np.float64), ora["scale"])
            T.compare_indices(T.host(b["idx"]).reshape(-1, n), T.u32(b["coset"]), ora, "E8",
                              n, "batch item %d" % i)
            yo = codec.bf16_rne(codec.decode(ora["idx"], ora["coset"], ora["scale"], "E8", n, 9))
            assert np.array_equal(T.bf16_host_bits(y).reshape(-1, n), codec.bf16_bits(yo)), i


def _pipeline_batches(rng, shapes, seed_bits):
    mats, hosts = [], []
    for r, c in shapes:
        w = rng.standard_normal((r, c)) * 0.02
        w[:, ::97] *= 400.0                       # a few outlier columns
        bits = workloads.f32_to_bf16_bits(w.astype(np.float32))
        hosts.append(workloads.bf16_bits_to_f64(bits))
        mats.append(T.bf16_device(bits, (r, c)))
    return mats, hosts


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_encode_decode_batch_matches_separate_calls(out_dtype):
    """hq_encode_decode_batch (one launch: encode of one batch interleaved
    with the decode of another) gives exactly the bytes of hq_encode_batch
    followed by hq_decode_batch: batches of different sizes and group counts
    (ragged tiles, an empty matrix), one side empty, and more than eight
    matrices (the two-launch fallback); the encode side also against the
    oracle on sampled tiles."""
    rng = np.random.default_rng(47)
    enc_shapes = [(7, 256), (33, 768), (0, 512), (5, 1024), (64, 256), (3, 2048)]
    dec_shapes = [(40, 256), (1, 512), (16, 1024), (9, 768)]
    emats, ehosts = _pipeline_batches(rng, enc_shapes, 0)
    dmats, _ = _pipeline_batches(rng, dec_shapes, 1)
    dsrc = hq.hq_encode_batch(dmats, "E8", 256, 4.0, 11)     # the layer to decode
    torch.cuda.synchronize()
    cases = [("both", emats, dsrc), ("encode only", emats, []), ("decode only", [], dsrc),
             ("nine + four (fallback)", emats + emats[:3], dsrc)]
    for label, em, ds in cases:
        say("case: pipeline %s, %s out" % (label, out_dtype))
        res, ys = hq.hq_encode_decode_batch(em, ds, "E8", 256, 4.0, enc_seed=5, dec_seed=11,
                                            out_dtype=out_dtype)
        ref_e = hq.hq_encode_batch(em, "E8", 256, 4.0, 5) if em else []
        ref_y = hq.hq_decode_batch(ds, "E8", 256, 11, out_dtype) if ds else []
        torch.cuda.synchronize()
        assert len(res) == len(ref_e) and len(ys) == len(ref_y)
        for i, (a, b) in enumerate(zip(res, ref_e)):
            for k in ("scale", "idx", "coset", "rice_k", "tile_bits"):
                assert torch.equal(a[k], b[k]), (label, i, k)
        for i, (a, b) in enumerate(zip(ys, ref_y)):
            assert torch.equal(a.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                               b.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)), \
                (label, i)
    # the encode side against the oracle (tiles every 7th)
    for i, h in enumerate(ehosts):
        if h.size == 0:
            continue
        tiles = np.arange(0, h.size // 256, 7)
        ora = codec.encode(codec.tiles(h, 256)[tiles], "E8", 256, 4.0, rht_seed=5)
        assert np.array_equal(T.host(res[i]["scale"]).reshape(-1)[tiles].astype(np.float64),
                              ora["scale"])
        T.compare_indices(T.host(res[i]["idx"]).reshape(-1, 256)[tiles],
                          T.u32(res[i]["coset"]).reshape(-1, 1)[tiles], ora, "E8", 256,
                          "pipeline encode item %d" % i)


def test_encode_decode_batch_refuses_overlap():
    """A decode batch that reads what the encode batch writes (or writes over
    its input) is refused before anything is enqueued."""
    rng = np.random.default_rng(3)
    mats, _ = _pipeline_batches(rng, [(8, 512)], 0)
    enc = hq.hq_encode_batch(mats, "E8", 256, 4.0, 1)
    torch.cuda.synchronize()
    with pytest.raises(hq.HQError) as e:          # decode reads the encode's own outputs
        hq.hq_encode_decode_batch(mats, enc, "E8", 256, 4.0, enc_seed=1, dec_seed=1, enc_outs=enc)
    assert e.value.code == hq.HQ_EINVAL
    other = hq.hq_encode_batch(mats, "E8", 256, 4.0, 2)
    with pytest.raises(hq.HQError) as e:          # decode writes over the encode's input
        hq.hq_encode_decode_batch(mats, other, "E8", 256, 4.0, dec_outs=[mats[0]])
    assert e.value.code == hq.HQ_EINVAL


def test_stack_sampled_parity_as_benchmarked():
    """The 32-layer Llama-3.1-8B-shaped stack exactly as bench.py runs it:
    each layer drawn on the GPU, one batched encode of its seven matrices and
    one batched decode (E8, tile 256, 4 bps, RHT seed = layer index).  Every
    257th tile of every matrix is copied to the host and checked against the
    oracle: scale, indices and cosets, Rice k and bits, and the decoded bf16
    of tiles whose indices match.  The counts over the 32 layers are printed
    and, when HQ_PARITY_RECORD names a file, appended to it."""
    dev = torch.device("cuda")
    stride = 257
    n_checked = 0
    tot = {"tiles": 0, "scale_skipped": 0, "blocks": 0, "mismatch": 0, "near_ties": 0}
    for layer in range(32):
        say("case: stack layer %d" % layer)
        xs = [workloads.llama_stack_torch(layer, m, dev) for m in range(len(workloads.LLAMA_LAYER))]
        encs = hq.hq_encode_batch(xs, "E8", 256, 4.0, layer)
        ys = hq.hq_decode_batch(encs, "E8", 256, layer, torch.bfloat16)
        torch.cuda.synchronize()
        parts = {k: [] for k in ("x", "scale", "idx", "coset", "rice_k", "tile_bits", "y")}
        for x, e, y in zip(xs, encs, ys):
            sel = torch.arange(0, x.numel() // 256, stride, device=dev)
            parts["x"].append(T.bf16_host_bits(x.view(-1, 256)[sel]))
            parts["scale"].append(T.host(e["scale"].view(-1)[sel]))
            parts["idx"].append(T.host(e["idx"].view(-1, 256)[sel]))
            parts["coset"].append(T.u32(e["coset"].view(-1, 1)[sel]))
            parts["rice_k"].append(T.host(e["rice_k"].view(-1)[sel]))
            parts["tile_bits"].append(T.u32(e["tile_bits"].view(-1)[sel]))
            parts["y"].append(T.bf16_host_bits(y.view(-1, 256)[sel]))
        del xs, encs, ys
        g = {k: np.concatenate(v) for k, v in parts.items()}
        X = workloads.bf16_bits_to_f64(g["x"]).reshape(-1, 256)
        ora = codec.encode(X, "E8", 256, 4.0, rht_seed=layer)
        skip = midpoint_close(oracle_pre_scale(X, "E8", 4.0))
        assert np.array_equal(g["scale"].astype(np.float64)[~skip], ora["scale"][~skip]), layer
        keep = np.nonzero(g["scale"].astype(np.float64) == ora["scale"])[0]
        sub = {k: (v[keep] if isinstance(v, np.ndarray) and v.shape[:1] == (len(X),) else v)
               for k, v in ora.items()}
        nbad, nnear, nblk, ok = T.compare_indices(g["idx"][keep], g["coset"][keep], sub, "E8", 256,
                                                  "stack layer %d" % layer)
        tot["tiles"] += len(X)
        tot["scale_skipped"] += int(np.sum(~(g["scale"].astype(np.float64) == ora["scale"])))
        tot["blocks"] += nblk
        tot["mismatch"] += nbad
        tot["near_ties"] += nnear
        assert np.array_equal(g["rice_k"][keep][ok].astype(np.int64), sub["rice_k"][ok]), layer
        assert np.array_equal(g["tile_bits"][keep][ok].astype(np.int64), sub["tile_bits"][ok]), layer
        yo = codec.bf16_rne(codec.decode(sub["idx"][ok], sub["coset"][ok], sub["scale"][ok],
                                         "E8", 256, layer))
        assert np.array_equal(g["y"][keep][ok].reshape(-1, 256), codec.bf16_bits(yo)), layer
        n_checked += len(X)
    say("stack: %d sampled tiles checked" % n_checked)
    rec = {"workload": "llama3.1-8b-shaped 32-layer stack as benchmarked (drawn on the GPU, "
                       "batched encode and bf16 decode per layer, RHT seed = layer), every "
                       "257th tile of every matrix", "lattice": "E8", "tile": 256, "bps": 4.0}
    rec.update(tot)
    rec.update({"near_tie_fraction": tot["near_ties"] / tot["blocks"],
                "mismatch_fraction": tot["mismatch"] / tot["blocks"]})
    say("  " + json.dumps(rec))
    path = os.environ.get("HQ_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def _stream_dev(words, off):
    w = torch.from_numpy(np.ascontiguousarray(words, np.uint32).view(np.int32)).cuda()
    if w.numel() == 0:
        w = torch.zeros(1, dtype=torch.int32, device="cuda")
    return w, torch.from_numpy(np.ascontiguousarray(off, np.int64)).cuda()


def _check_unpacked(g, idx, coset_rows, k, lattice, n, label):
    assert np.array_equal(T.host(g["idx"]).astype(np.int64), idx), label + " idx"
    assert np.array_equal(T.host(g["rice_k"]).astype(np.int64), k), label + " k"
    if coset_rows.shape[1]:
        from oracle import rice
        got = rice.coset_bit_rows(T.u32(g["coset"]), coset_rows.shape[1])
        assert np.array_equal(got, coset_rows), label + " coset"


@pytest.mark.parametrize("lattice,n", [("E8", 256), ("E8", 128), ("D4", 128), ("A2", 128),
                                       ("A2", 256), ("Z", 256), ("E8", 64), ("E8", 512),
                                       ("A2", 512), ("D4", 64)])
def test_unpack_parity(lattice, n):
    """hq_unpack of the oracle's packed stream gives the oracle's indices,
    coset bits and k (oracle unpack of the same words), on a ragged tile
    count; hq_unpack of the GPU's own packed stream gives back the indices."""
    from oracle import rice
    rows, cols = 37, 6 * n          # 222 tiles: not a multiple of 64
    rng = np.random.default_rng(41)
    w = rng.standard_normal((rows, cols)) * 0.02
    w[:, 3] *= 200.0
    xh = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(w.astype(np.float32)))
    cb = codec.coset_bits_per_tile(lattice, n)
    for bps in (2.0, 4.0):
        label = "unpack %s/%d R=%g" % (lattice, n, bps)
        say("case:", label)
        ora = codec.encode(xh, lattice, n, bps, rht_seed=7)
        k, tb, total, words, off = codec.rate(ora["idx"], ora["coset"], lattice, n)
        ref_idx, ref_cos, ref_k = rice.unpack(words, off, n, cb)
        assert np.array_equal(ref_idx, ora["idx"])          # the oracle's own round trip
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        wd, od = _stream_dev(words, off)
        g = hq.hq_unpack(wd, od, lattice, n, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0, label
        _check_unpacked(g, ref_idx, ref_cos, ref_k, lattice, n, label)
        # the GPU's own pack, unpacked on the GPU
        cw = ora["coset"].astype(np.uint32)
        r = hq.hq_rate(torch.from_numpy(ora["idx"].astype(np.int8)).cuda(),
                       torch.from_numpy(cw.view(np.int32)).cuda() if cw.size else None,
                       lattice, n, pack=True)
        g2 = hq.hq_unpack(r["stream"], r["tile_word_offset"], lattice, n, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0, label
        _check_unpacked(g2, ref_idx, ref_cos, ref_k, lattice, n, label + " (gpu pack)")


@pytest.mark.parametrize("lattice,n", [("E8", 256), ("A2", 128)])
def test_unpack_batch_matches_oracle_and_single_calls(lattice, n):
    """hq_unpack_batch over eleven packed matrices (more than one launch of
    eight, one empty, ragged tile counts from 1 to 1300): each item gives
    the oracle's indices, coset bits and k, the same bytes as one hq_unpack
    call, and an empty item is skipped."""
    from oracle import rice
    rng = np.random.default_rng(53)
    cb = codec.coset_bits_per_tile(lattice, n)
    counts = [7, 0, 64, 65, 300, 1, 129, 1300, 33, 200, 2]
    packs, refs = [], []
    for i, nt in enumerate(counts):
        if nt == 0:
            refs.append(None)
            packs.append({"stream": torch.zeros(1, dtype=torch.int32, device="cuda"),
                          "tile_word_offset": torch.zeros(1, dtype=torch.int64, device="cuda")})
            continue
        w = rng.standard_normal((nt, n)) * 0.02
        w[:, 5] *= 100.0
        xh = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(w.astype(np.float32)))
        ora = codec.encode(xh, lattice, n, 3.0 + (i % 3), rht_seed=i)
        k, tb, total, words, off = codec.rate(ora["idx"], ora["coset"], lattice, n)
        refs.append(rice.unpack(words, off, n, cb))
        wd, od = _stream_dev(words, off)
        packs.append({"stream": wd, "tile_word_offset": od})
    say("case: unpack batch of %d matrices, %s/%d" % (len(counts), lattice, n))
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = hq.hq_unpack_batch(packs, lattice, n, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, (g, ref) in enumerate(zip(got, refs)):
        if ref is None:
            assert g["idx"].numel() == 0
            continue
        _check_unpacked(g, ref[0], ref[1], ref[2], lattice, n, "batch item %d" % i)
        one = hq.hq_unpack(packs[i]["stream"], packs[i]["tile_word_offset"], lattice, n)
        torch.cuda.synchronize()
        assert torch.equal(one["idx"], g["idx"]) and torch.equal(one["rice_k"], g["rice_k"]), i
        if cb:
            assert torch.equal(one["coset"], g["coset"]), i


def _forced_k_stream(idx, coset_rows, ks):
    """Packed words of tiles coded with the given k (not the optimal one),
    through the oracle's own tile bit-string writer."""
    from oracle import rice
    segs, off = [], [0]
    for t in range(idx.shape[0]):
        bits = rice._tile_bitstring(idx[t], coset_rows[t], int(ks[t]))
        nwords = (bits.size + 31) // 32
        padded = np.zeros(nwords * 32, np.uint8)
        padded[:bits.size] = bits
        segs.append(np.packbits(padded, bitorder="little").view("<u4"))
        off.append(off[-1] + nwords)
    return np.concatenate(segs).astype(np.uint32), np.asarray(off, np.int64)


def test_unpack_any_k_long_codes_and_corrupt_tiles():
    """Streams whose tiles use any k in 0..15 (long unary runs at k = 0,
    wide remainders at k = 15) decode as the oracle's unpack does; a tile
    whose words end early, or whose word range is reversed, sets
    HQ_ST_CORRUPT without disturbing the other tiles."""
    from oracle import rice
    rng = np.random.default_rng(43)
    n, nt = 256, 70
    idx = rng.integers(-128, 128, size=(nt, n))
    idx[::3] = rng.integers(-3, 4, size=idx[::3].shape)
    cos = rng.integers(0, 2, size=(nt, 32)).astype(np.uint8)
    ks = np.arange(nt) % 16
    words, off = _forced_k_stream(idx, cos, ks)
    ref_idx, ref_cos, ref_k = rice.unpack(words, off, n, 32)
    assert np.array_equal(ref_idx, idx) and np.array_equal(ref_k, ks)
    say("case: unpack forced k 0..15")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    wd, od = _stream_dev(words, off)
    g = hq.hq_unpack(wd, od, "E8", n, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    _check_unpacked(g, ref_idx, ref_cos, ref_k, "E8", n, "forced k")
    # last tile three words short; tile 9's range reversed (which also
    # moves the start of tile 10)
    say("case: unpack corrupt tiles")
    bad_off = off.copy()
    bad_off[-1] -= 3
    bad_off[10] = bad_off[9] - 1
    wd, od = _stream_dev(words, bad_off)
    st.zero_()
    g = hq.hq_unpack(wd, od, "E8", n, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & hq.HQ_ST_CORRUPT
    good = np.ones(nt, bool)
    good[[9, 10, nt - 1]] = False       # tile 10 now starts inside tile 8
    assert np.array_equal(T.host(g["idx"]).astype(np.int64)[good], idx[good])


@pytest.mark.parametrize("lattice,n", [("E8", 256), ("A2", 128), ("D4", 64)])
def test_rate_batch_matches_single_calls(lattice, n):
    """hq_rate_batch on ten matrices of mixed sizes (one tile, ragged counts,
    more than one launch group), rate only, packing, and packing with the
    encoder's values given: every output equals one hq_rate call per
    matrix, bit for bit (streams up to their last word)."""
    rng = np.random.default_rng(91 + n)
    shapes = [(1, n), (37, 1536), (300, 4096), (5, 768), (129, 2048), (64, 512), (2, 4096),
              (1000, 1024), (3, 256), (90, 2560)]
    encs = []
    for i, (rows, cols) in enumerate(shapes):
        bits = workloads.f32_to_bf16_bits((rng.standard_normal((rows, cols)) * 0.02)
                                          .astype(np.float32))
        encs.append(hq.hq_encode_tiles(T.bf16_device(bits, (rows, cols)), lattice, n, 4.0, 3))
    for pack, given in ((False, False), (True, False), (True, True)):
        say("case: rate batch %s/%d pack=%s given=%s" % (lattice, n, pack, given))
        batch = hq.hq_rate_batch(encs, lattice, n, pack=pack, given=given)
        for i, e in enumerate(encs):
            one = hq.hq_rate(e["idx"], e["coset"], lattice, n, pack=pack,
                             given=e if given else None)
            torch.cuda.synchronize()
            b = batch[i]
            assert torch.equal(b["rice_k"], one["rice_k"]), i
            assert torch.equal(b["tile_bits"], one["tile_bits"]), i
            assert int(b["total_bits"].item()) == int(one["total_bits"].item()), i
            if pack:
                assert torch.equal(b["tile_word_offset"], one["tile_word_offset"]), i
                nw = int(one["tile_word_offset"][-1].item())
                assert torch.equal(b["stream"][:nw], one["stream"][:nw]), i


def test_rate_given_values_that_do_not_hold_the_codes():
    """HQ_RATE_GIVEN with rice_k / tile_bits that are not the encoder's: a k
    above 8, a k one below the optimum (longer codes than tile_bits), and
    tile_bits past what a tile can need.  Those tiles set HQ_ST_CORRUPT and
    leave their codes unwritten; every other tile's words are the oracle's."""
    rng = np.random.default_rng(47)
    n, nt = 256, 60
    x = rng.standard_normal((nt, n))
    bits = workloads.f32_to_bf16_bits(x.astype(np.float32))
    ora = codec.encode(workloads.bf16_bits_to_f64(bits), "E8", n, 4.0, rht_seed=2)
    k, tb, total, words, off = codec.rate(ora["idx"], ora["coset"], "E8", n)
    gk, gtb = k.copy(), tb.copy()
    j = int(np.nonzero(k >= 1)[0][3])
    gk[7] = 12                                   # k above 8
    gk[j] = k[j] - 1                             # first minimum: k - 1 costs more
    gtb[40] = 1 << 20                            # past any tile's words
    idx = torch.from_numpy(ora["idx"].astype(np.int8)).cuda()
    coset = torch.from_numpy(ora["coset"].astype(np.uint32).view(np.int32)).cuda()
    given = {"rice_k": torch.from_numpy(gk.astype(np.uint8)).cuda(),
             "tile_bits": torch.from_numpy(gtb.astype(np.uint32).view(np.int32)).cuda()}
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("case: rate with given values that do not hold the codes")
    r = hq.hq_rate(idx, coset, "E8", n, pack=True, given=given, status=st,
                   capacity_words=int(off[-1]) + (1 << 16))
    torch.cuda.synchronize()
    assert int(st.item()) & hq.HQ_ST_CORRUPT
    goff = T.host(r["tile_word_offset"])
    gw = T.u32(r["stream"])
    bad = {7, j, 40}
    for t in range(nt):
        if t in bad:
            continue
        w = gw[goff[t]:goff[t] + (off[t + 1] - off[t])]
        assert np.array_equal(w, words[off[t]:off[t + 1]]), t


@pytest.mark.parametrize("m", [1, 3, 8])
def test_gemv_parity(m):
    """hq_gemv against the oracle: y = W x with W the oracle's fp64 decode of
    the oracle's own encode (a ragged 37 x 1536 matrix and a Llama-shaped k
    projection, 1024 x 4096, RHT seed 5), x seeded N(0, 1) in fp32.  Bound
    for fp32: a product passes at most 1 rounding of the rotated input, 9 of
    the block's multiply-add chain, 2 adding the coset term and the second
    block, 1 of the scale, (pieces - 1) adding a lane's 1024-column pieces,
    6 of the 64-lane sum and (chunks - 1) of the chunk sum: 17 + pieces +
    chunks in all, at most 22 here (pieces + chunks <= 5 for 6 and 16
    slices at every m), so |y - y_ref| <= (slices + 16) 2^-24 B with
    B = sum_t Delta/32 sum_j |P_j| |(H (s . x_t))_j|, computed here in fp64."""
    from oracle import hadamard, splitmix
    rng = np.random.default_rng(51 + m)
    for rows, cols in ((37, 1536), (1024, 4096)):
        label = "gemv %dx%d m=%d" % (rows, cols, m)
        say("case:", label)
        w = rng.standard_normal((rows, cols)) * 0.02
        w[:, 7] *= 50.0
        xh = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(w.astype(np.float32)))
        ora = codec.encode(xh, "E8", 256, 4.0, rht_seed=5)
        W = codec.decode(ora["idx"], ora["coset"], ora["scale"], "E8", 256, 5).reshape(rows, cols)
        x = rng.standard_normal((m, cols)).astype(np.float32)
        y_ref = x.astype(np.float64) @ W.T                                  # (m, rows)
        T_ = cols // 256
        P = np.abs(ora["coords"].reshape(rows, T_, 256).astype(np.float64))
        signs = splitmix.rht_signs(5, 256)
        xr = np.abs(hadamard.unnormalized_forward(x.astype(np.float64).reshape(m * T_, 256),
                                                  signs)).reshape(m, T_, 256)
        dl = ora["scale"].reshape(rows, T_) / 32.0
        B = np.einsum("rt,rtj,vtj->vr", dl, P, xr)
        tol = (T_ + 16) * 2.0 ** -24 * B
        idx = torch.from_numpy(ora["idx"].astype(np.int8).reshape(rows, cols)).cuda()
        cw = torch.from_numpy(ora["coset"].astype(np.uint32).view(np.int32)).cuda()
        sc = torch.from_numpy(ora["scale"].astype(np.float32)).cuda()
        y = hq.hq_gemv(idx, cw, sc, torch.from_numpy(x).cuda(), rht_seed=5)
        torch.cuda.synchronize()
        err = np.abs(T.host(y).astype(np.float64) - y_ref)
        assert np.all(err <= tol), "%s: max err/tol %.3g" % (label, np.max(err / tol))
        # one vector as a 1-D input
        y1 = hq.hq_gemv(idx, cw, sc, torch.from_numpy(x[0]).cuda(), rht_seed=5)
        torch.cuda.synchronize()
        assert np.all(np.abs(T.host(y1) - y_ref[0]) <= tol[0]), label + " 1-D"


def _gemm_case(rng, rows, cols, m, seed):
    """An oracle-encoded E8/256 matrix (N(0, 0.02^2) with a planted column),
    m seeded N(0, 1) fp32 inputs, the fp64 product with the oracle's decode
    and the error bound of the GPU GEMM.  Bound: the two bf16 terms of a
    rotated input miss it by at most 2^-16 of its size; the exact products
    accumulate in fp32 inside the matrix core (at most 64 roundings per
    slice: 32 products of the slice per output pass through two chains of
    16 steps), then one rounding of the scale and one per slice sum and per
    range sum, so |y - y_ref| <= (2^-16 + (slices + 80) 2^-24) B with
    B = sum_t Delta/32 sum_j |P_j| |(H (s . x_t))_j| in fp64."""
    from oracle import hadamard, splitmix
    w = rng.standard_normal((rows, cols)) * 0.02
    w[:, 7] *= 50.0
    xh = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(w.astype(np.float32)))
    ora = codec.encode(xh, "E8", 256, 4.0, rht_seed=seed)
    W = codec.decode(ora["idx"], ora["coset"], ora["scale"], "E8", 256, seed).reshape(rows, cols)
    x = rng.standard_normal((m, cols)).astype(np.float32)
    y_ref = x.astype(np.float64) @ W.T                                  # (m, rows)
    T_ = cols // 256
    P = np.abs(ora["coords"].reshape(rows, T_, 256).astype(np.float64))
    xr = np.abs(hadamard.unnormalized_forward(x.astype(np.float64).reshape(m * T_, 256),
                                              splitmix.rht_signs(seed, 256))).reshape(m, T_, 256)
    B = np.einsum("rt,rtj,vtj->vr", ora["scale"].reshape(rows, T_) / 32.0, P, xr)
    tol = (2.0 ** -16 + (T_ + 80) * 2.0 ** -24) * B
    enc = {"idx": torch.from_numpy(ora["idx"].astype(np.int8).reshape(rows, cols)).cuda(),
           "coset": torch.from_numpy(ora["coset"].astype(np.uint32).view(np.int32)).cuda(),
           "scale": torch.from_numpy(ora["scale"].astype(np.float32)).cuda()}
    return enc, torch.from_numpy(x).cuda(), y_ref, tol


@pytest.mark.parametrize("m", [1, 5, 32, 33, 64, 100, 200, 300])
def test_gemm_parity(m):
    """hq_gemm against the oracle: Y = X W^T with W the oracle's fp64 decode
    of the oracle's own encode (ragged 37 x 1536, 300 x 768 and a Llama-shaped
    k projection 1024 x 4096, RHT seed 5), m vectors (one and two 32-vector
    fragments per block, the 128-vector wide tiles above 192, several and
    ragged vector blocks), within the bound of _gemm_case.  Two calls give
    the same bits."""
    rng = np.random.default_rng(61 + m)
    for rows, cols in ((37, 1536), (300, 768), (1024, 4096)):
        label = "gemm %dx%d m=%d" % (rows, cols, m)
        say("case:", label)
        enc, xd, y_ref, tol = _gemm_case(rng, rows, cols, m, 5)
        y = hq.hq_gemm(enc["idx"], enc["coset"], enc["scale"], xd, rht_seed=5)
        y2 = hq.hq_gemm(enc["idx"], enc["coset"], enc["scale"], xd, rht_seed=5)
        torch.cuda.synchronize()
        err = np.abs(T.host(y).astype(np.float64) - y_ref)
        assert np.all(err <= tol), "%s: max err/tol %.3g" % (label, np.max(err / tol))
        assert torch.equal(y, y2), label + " determinism"


@pytest.mark.parametrize("m", [3, 40, 130, 260])
def test_gemm_batch_parity(m):
    """hq_gemm_batch on ten oracle-encoded matrices of mixed shapes (ragged
    row counts, one and many slices, split and unsplit slice ranges; two
    launch groups) against the oracle, each within the bound of _gemm_case;
    a second call gives the same bits."""
    rng = np.random.default_rng(71 + m)
    shapes = [(37, 1536), (64, 4096), (5, 256), (40, 14336), (129, 2048), (1, 768),
              (600, 512), (256, 1024), (3, 4096), (90, 512)]
    cases = []
    for i, (rows, cols) in enumerate(shapes):
        say("case: gemm batch m=%d item %d %dx%d" % (m, i, rows, cols))
        cases.append(_gemm_case(rng, rows, cols, m, 9))
    mats = [c[0] for c in cases]
    xs = [c[1] for c in cases]
    ys = hq.hq_gemm_batch(mats, xs, rht_seed=9)
    ys2 = hq.hq_gemm_batch(mats, xs, rht_seed=9)
    torch.cuda.synchronize()
    for i, (enc, xd, y_ref, tol) in enumerate(cases):
        err = np.abs(T.host(ys[i]).astype(np.float64) - y_ref)
        assert np.all(err <= tol), "item %d %s: max err/tol %.3g" % (i, shapes[i],
                                                                     np.max(err / tol))
        assert torch.equal(ys[i], ys2[i]), "item %d determinism" % i


def test_layer_gemm_and_gemv_as_benchmarked():
    """The Llama-3.1-8B-shaped layer as bench.py runs its products: the seven
    matrices drawn on the GPU and encoded in one batch (E8/256, 4 bps, RHT
    seed 0), then hq_gemm_batch at m = 32, 128 and 256 and hq_gemv_batch at
    m = 1.
    Property checked at this size: each product equals X W^T for the fp32
    weights hq_decode_tiles gives, within the GEMM bound
    (2^-16 + (slices + 80) 2^-24) B plus the fp32 decode's rounding
    2^-23 |X| |W|^T, where B <= sum_t |w_rt| |x_vt| (per 256-column tile:
    Delta / 32 <|P|, |H (s . x)|> is at most the product of the tile norms,
    the rotation being orthonormal up to the factor the norms carry)."""
    dev = torch.device("cuda")
    xs = [workloads.llama_stack_torch(0, m, dev) for m in range(len(workloads.LLAMA_LAYER))]
    encs = hq.hq_encode_batch(xs, "E8", 256, 4.0, 0)
    del xs
    ws = [hq.hq_decode_tiles(e["idx"], e["coset"], e["scale"], "E8", 256, 0, torch.float32)
          for e in encs]
    gen = torch.Generator(device=dev)
    gen.manual_seed(23)
    for m in (32, 128, 256, 1):
        say("case: layer products m=%d" % m)
        xm = [torch.randn(m, w.shape[1], device=dev, generator=gen) for w in ws]
        if m == 1:
            ys = hq.hq_gemv_batch(encs, xm, rht_seed=0)
        else:
            ys = hq.hq_gemm_batch(encs, xm, rht_seed=0)
        torch.cuda.synchronize()
        for i, (w, x, y) in enumerate(zip(ws, xm, ys)):
            w64, x64 = w.double(), x.double()
            ref = x64 @ w64.t()
            T_ = w.shape[1] // 256
            wn = w64.view(w.shape[0], T_, 256).norm(dim=2)           # (rows, tiles)
            xn = x64.view(m, T_, 256).norm(dim=2)                    # (m, tiles)
            tol = (2.0 ** -16 + (T_ + 80) * 2.0 ** -24) * (xn @ wn.t()) + \
                2.0 ** -23 * (x64.abs() @ w64.abs().t())
            err = (y.double().view(m, -1) - ref).abs()
            worst = float((err / tol).max())
            say("  matrix %d %s: max err/tol %.3g" % (i, tuple(w.shape), worst))
            assert worst <= 1.0, "m=%d matrix %d" % (m, i)


@pytest.mark.parametrize("m", [1, 2, 3])
def test_gemv_batch_matches_single_calls(m):
    """hq_gemv_batch on ten matrices of mixed shapes (ragged row counts, one
    and several column chunks per row; more than one launch group) gives
    each matrix's hq_gemv result bit for bit."""
    rng = np.random.default_rng(61 + m)
    shapes = [(37, 1536), (64, 4096), (5, 256), (300, 14336), (129, 2048), (1, 768),
              (77, 5120), (256, 1024), (3, 4096), (90, 512)]
    mats, xs = [], []
    for i, (rows, cols) in enumerate(shapes):
        w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
        bits = workloads.f32_to_bf16_bits(w)
        say("case: gemv batch m=%d item %d %dx%d" % (m, i, rows, cols))
        mats.append(hq.hq_encode_tiles(T.bf16_device(bits, (rows, cols)), "E8", 256, 4.0, 9))
        x = rng.standard_normal((m, cols)).astype(np.float32)
        xs.append(torch.from_numpy(x[0] if m == 1 else x).cuda())
    ys = hq.hq_gemv_batch(mats, xs, rht_seed=9)
    torch.cuda.synchronize()
    for i, (e, x) in enumerate(zip(mats, xs)):
        y1 = hq.hq_gemv(e["idx"], e["coset"], e["scale"], x, rht_seed=9)
        torch.cuda.synchronize()
        assert np.array_equal(T.host(ys[i]).view(np.uint32), T.host(y1).view(np.uint32)), i


@pytest.mark.parametrize("dither", [True, False])
def test_kv_scores_parity(dither):
    """hq_kv_scores against the oracle: q . khat with khat the oracle's fp64
    decode (dither subtracted) of the oracle's encode of 300 seeded keys
    (not a multiple of the 256 keys of a block; dither base 1000) for 40
    queries (a full and a ragged chunk of 32).  Bound for fp32: each product
    q~_i yhat_i passes through at most 136 roundings (the rotated query,
    yhat's difference and scale, the 128-term sums, the final 1/sqrt(128)),
    so |s - s_ref| <= 136 2^-24 sum_i |q~_i| |yhat_i| / sqrt(128), with
    q~ = H (s . q) and yhat = Delta (p - d) computed here in fp64."""
    from oracle import hadamard, splitmix
    rng = np.random.default_rng(61 + int(dither))
    nk, nq, base = 300, 40, 1000
    k = rng.standard_normal((nk, 128))
    k[:, [3, 77]] += 4.0                                # channel offsets
    xh = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(k.astype(np.float32)))
    ds = 2 if dither else None
    say("case: kv scores dither=%s" % dither)
    ora = codec.encode(xh, "E8", 128, 4.0, rht_seed=1, dither_seed=ds, dither_base=base)
    khat = codec.decode(ora["idx"], ora["coset"], ora["scale"], "E8", 128, 1,
                        dither_seed=ds, dither_base=base)
    q = rng.standard_normal((nq, 128)).astype(np.float32)
    ref = q.astype(np.float64) @ khat.T
    p = codec.lattice_points(ora["idx"], ora["coset"], "E8", 128)
    if dither:
        p = p - codec.dither(ds, base, nk, 128)
    yhat = ora["scale"][:, None] * p
    qr = hadamard.unnormalized_forward(q.astype(np.float64), splitmix.rht_signs(1, 128))
    tol = 136 * 2.0 ** -24 * (np.abs(qr) @ np.abs(yhat).T) / math.sqrt(128.0)
    enc = {"idx": torch.from_numpy(ora["idx"].astype(np.int8)).cuda(),
           "coset": torch.from_numpy(ora["coset"].astype(np.uint32).view(np.int32)).cuda(),
           "scale": torch.from_numpy(ora["scale"].astype(np.float32)).cuda()}
    g = hq.hq_kv_scores(torch.from_numpy(q).cuda(), enc, rht_seed=1, dither_seed=ds,
                        dither_base=base)
    torch.cuda.synchronize()
    err = np.abs(T.host(g).astype(np.float64) - ref)
    assert np.all(err <= tol), "max err/tol %.3g" % np.max(err / tol)


@pytest.mark.parametrize("bps", [1.7, 2.5])
def test_kv_low_rate_parity(bps):
    """Low-rate KV operating points: 2048 K vectors (128, bf16, channel
    offsets) encoded with the dither at 1.7 and 2.5 bps against the oracle
    (every vector), and the dithered decode bit-exact against the oracle's."""
    rng = np.random.default_rng(71)
    k = rng.standard_normal((2048, 128))
    k[:, [5, 90]] += 3.0
    bits = workloads.f32_to_bf16_bits(k.astype(np.float32))
    xh = workloads.bf16_bits_to_f64(bits)
    say("case: kv low rate %g bps" % bps)
    g = hq.hq_kv_encode(T.bf16_device(bits, (2048, 128)), bps, 1, dither_seed=9, dither_base=77)
    torch.cuda.synchronize()
    ora = codec.encode(xh, "E8", 128, bps, rht_seed=1, dither_seed=9, dither_base=77)
    assert np.array_equal(T.host(g["scale"]).astype(np.float64), ora["scale"])
    _, _, _, ok = T.compare_indices(T.host(g["idx"]), T.u32(g["coset"]), ora, "E8", 128,
                                    "kv %g bps" % bps)
    assert np.array_equal(T.host(g["rice_k"])[ok].astype(np.int64), ora["rice_k"][ok])
    assert np.array_equal(T.u32(g["tile_bits"])[ok].astype(np.int64), ora["tile_bits"][ok])
    check_decode(ora, "E8", 128, 1, "kv %g bps" % bps, exact=True, dither_seed=9, dither_base=77)


@pytest.mark.parametrize("lattice,n,dtype,bps", [("E8", 256, "bf16", 4.0), ("E8", 256, "bf16", 2.0),
                                                 ("E8", 256, "bf16", 3.0), ("E8", 256, "bf16", 5.0),
                                                 ("E8", 128, "f32", 3.0),
                                                 ("D4", 128, "bf16", 4.0), ("A2", 64, "bf16", 3.5),
                                                 ("Z", 512, "f32", 5.0)])
def test_rate_control_parity(lattice, n, dtype, bps):
    """Per-tile rate control (bisection on bf16 scales to floor(bps n) bits per
    tile) against the oracle on a ragged matrix with outlier columns: the
    chosen scales bit for bit, indices, k and bits, and every tile within
    its budget; then the decoded values.  E8/256 bf16 runs on the fast
    kernel, and again on the generic one (a call that exports coordinates),
    with the same results."""
    rows, cols = 29, 5 * n
    rng = np.random.default_rng(97)
    w = rng.standard_normal((rows, cols)) * 0.02
    w[:, 2] *= 80.0
    w[3] = 0.0
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(w.astype(np.float32))
        xh = workloads.bf16_bits_to_f64(bits)
        xd = T.bf16_device(bits, (rows, cols))
    else:
        xh = w.astype(np.float32)
        xd = T.f32_device(xh)
    label = "rate control %s/%d %s R=%g" % (lattice, n, dtype, bps)
    say("case:", label)
    g = hq.hq_encode_tiles(xd, lattice, n, bps, 4, rate_control=True)
    torch.cuda.synchronize()
    ora = codec.encode(xh, lattice, n, bps, rht_seed=4, rate_control=True)
    assert np.array_equal(T.host(g["scale"]).astype(np.float64), ora["scale"]), label
    _, _, _, ok = T.compare_indices(T.host(g["idx"]).reshape(-1, n), T.u32(g["coset"]), ora,
                                    lattice, n, label)
    assert ok.all()
    assert np.array_equal(T.host(g["rice_k"]).astype(np.int64), ora["rice_k"])
    gb = T.u32(g["tile_bits"]).astype(np.int64)
    assert np.array_equal(gb, ora["tile_bits"])
    assert np.all(gb <= math.floor(bps * n))
    check_decode(ora, lattice, n, 4, label, exact=(lattice != "A2"))
    if (lattice, n, dtype) == ("E8", 256, "bf16"):
        gg = hq.hq_encode_tiles(xd, lattice, n, bps, 4, rate_control=True, want_coords=True)
        torch.cuda.synchronize()
        for key in ("scale", "idx", "coset", "rice_k", "tile_bits"):
            assert torch.equal(gg[key], g[key]), label + " generic vs fast " + key


def test_kv_head_dim_64_dither_parity():
    """Dithered E8 encode and decode of 300 KV vectors of 64 (tile 64,
    generic kernels) against the oracle, every vector."""
    rng = np.random.default_rng(83)
    x = rng.standard_normal((300, 64))
    x[:, 3] += 2.0
    bits = workloads.f32_to_bf16_bits(x.astype(np.float32))
    xh = workloads.bf16_bits_to_f64(bits)
    say("case: kv head dim 64, dither")
    g = hq.hq_kv_encode(T.bf16_device(bits, (300, 64)), 4.0, 2, dither_seed=5, dither_base=40)
    torch.cuda.synchronize()
    ora = codec.encode(xh, "E8", 64, 4.0, rht_seed=2, dither_seed=5, dither_base=40)
    skip = midpoint_close(oracle_pre_scale(xh, "E8", 4.0))
    assert not skip.any()
    assert np.array_equal(T.host(g["scale"]).astype(np.float64), ora["scale"])
    _, _, _, ok = T.compare_indices(T.host(g["idx"]), T.u32(g["coset"]), ora, "E8", 64, "kv 64")
    assert np.array_equal(T.host(g["rice_k"])[ok].astype(np.int64), ora["rice_k"][ok])
    assert np.array_equal(T.u32(g["tile_bits"])[ok].astype(np.int64), ora["tile_bits"][ok])
    check_decode(ora, "E8", 64, 2, "kv 64", exact=True, dither_seed=5, dither_base=40)


def test_e8_128_groups_edges():
    """E8 / tile 128 on the edges of its 32-vector groups: dithered encodes
    of 1, 31, 33 and 95 vectors (a zero vector among them) at dither offsets
    up to 2^31; caller scales (arbitrary fp32 values); decode of arbitrary
    int8 indices, whose Hadamard sums leave the int16 range, with and without
    the dither; the status bits."""
    rng = np.random.default_rng(41)
    for nvec, base in ((1, 5), (31, 1000), (33, 77777), (95, 2 ** 31)):
        x = rng.standard_normal((nvec, 128)) * 0.5 + 0.1
        x[nvec // 2] = 0.0
        bits = workloads.f32_to_bf16_bits(x.astype(np.float32))
        xh = workloads.bf16_bits_to_f64(bits)
        label = "kv %d vectors, dither base %d" % (nvec, base)
        say("case:", label)
        g = hq.hq_kv_encode(T.bf16_device(bits, (nvec, 128)), 4.0, 3, dither_seed=9,
                            dither_base=base)
        torch.cuda.synchronize()
        ora = codec.encode(xh, "E8", 128, 4.0, rht_seed=3, dither_seed=9, dither_base=base)
        skip = midpoint_close(oracle_pre_scale(xh, "E8", 4.0))
        assert not skip.any()
        assert np.array_equal(T.host(g["scale"]).astype(np.float64), ora["scale"]), label
        _, _, _, ok = T.compare_indices(T.host(g["idx"]), T.u32(g["coset"]), ora, "E8", 128,
                                        label)
        assert np.array_equal(T.host(g["rice_k"])[ok].astype(np.int64), ora["rice_k"][ok])
        assert np.array_equal(T.u32(g["tile_bits"])[ok].astype(np.int64), ora["tile_bits"][ok])
        check_decode(ora, "E8", 128, 3, label, exact=True, dither_seed=9, dither_base=base)

    # caller scales: the automatic ones times 1.37, rounded to fp32
    x = rng.standard_normal((70, 128))
    bits = workloads.f32_to_bf16_bits(x.astype(np.float32))
    xh = workloads.bf16_bits_to_f64(bits)
    sc = (codec.encode(xh, "E8", 128, 4.0, rht_seed=3)["scale"] * 1.37).astype(np.float32)
    ora = codec.encode(xh, "E8", 128, 4.0, rht_seed=3, scale=sc.astype(np.float64))
    say("case: E8/128 caller scales")
    g = hq.hq_encode_tiles(T.bf16_device(bits, (70, 128)), "E8", 128, 4.0, 3,
                           scale=torch.from_numpy(sc).cuda())
    torch.cuda.synchronize()
    _, _, _, ok = T.compare_indices(T.host(g["idx"]), T.u32(g["coset"]), ora, "E8", 128,
                                    "caller scales")
    assert np.array_equal(T.host(g["rice_k"])[ok].astype(np.int64), ora["rice_k"][ok])
    assert np.array_equal(T.u32(g["tile_bits"])[ok].astype(np.int64), ora["tile_bits"][ok])
    check_decode(ora, "E8", 128, 3, "caller scales", exact=True)

    # arbitrary indices (bf16-valued scales keep every product exact)
    n = 45
    idx = rng.integers(-128, 128, size=(n, 128))
    idx[0], idx[1] = 127, -128
    idx[2:20] = rng.integers(-3, 4, size=(18, 128))
    cw = rng.integers(0, 2 ** 16, size=(n, 1)).astype(np.uint32)
    scale = codec.bf16_rne(2.0 ** rng.uniform(-8, 2, size=n))
    arb = {"idx": idx, "coset": cw, "scale": scale}
    say("case: E8/128 arbitrary indices")
    check_decode(arb, "E8", 128, 5, "arbitrary indices", exact=True)
    check_decode(arb, "E8", 128, 5, "arbitrary indices, dither", exact=True, dither_seed=4,
                 dither_base=123)

    # status bits
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv = torch.randn((40, 128), device="cuda").to(torch.bfloat16)
    kv[33, 100] = float("inf")
    hq.hq_kv_encode(kv, 4.0, 0, dither_seed=1, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & hq.HQ_ST_NONFINITE
    st.zero_()
    hq.hq_encode_tiles(kv[:32].contiguous(), "E8", 128, 4.0, 0,
                       scale=torch.full((32,), 1e-4, device="cuda"), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == hq.HQ_ST_OVERFLOW


@pytest.mark.parametrize("lattice,n", [("E8", 128), ("D4", 128), ("A2", 128), ("Z", 128),
                                       ("E8", 256)])
def test_fast_grid_clamp(lattice, n):
    """Caller scales near the grid clamp: bf16 input (the tile-128 and the
    E8 / tile-256 fast kernels) against fp32 input of the same values (the
    generic kernel) and the oracle.  A tile A (s * h_k) (signs times Hadamard row k)
    rotates to one coordinate of size ||x|| / Delta, so its scale puts the
    largest grid value where wanted: HQ_ST_OVERFLOW is set iff some oracle
    grid value passes 124 (the clamp), and the other tiles of the call, which
    share the clamped grid of the spike's wave, match the oracle."""
    from oracle import hadamard, splitmix
    seed, bps = 3, 4.0
    s = splitmix.rht_signs(seed, n)
    H = hadamard.sylvester(n)
    rng = np.random.default_rng(17)
    for target in (123.5, 124.0 + 2.0 ** -20, 124.4, 125.9, 126.6, 131.0):
        x = rng.standard_normal((40, n)) * 0.02
        x[9] = s * H[77]                       # ||x|| = sqrt(n), one rotated coordinate
        bits = workloads.f32_to_bf16_bits(x.astype(np.float32))
        xh = workloads.bf16_bits_to_f64(bits)
        sc = codec.auto_scale(xh, lattice, bps).astype(np.float32)
        sc[9] = np.float32(math.sqrt(n) / target)
        ora = codec.encode(xh, lattice, n, bps, rht_seed=seed, scale=sc.astype(np.float64))
        U = np.rint(ora["u"] * 2.0 ** 24)
        flagged = bool(np.any(np.abs(U) > 124 * 2 ** 24))
        label = "%s/%d spike |u| = %g" % (lattice, n, target)
        say("case:", label, "flag expected" if flagged else "no flag")
        res = []
        for xd in (T.bf16_device(bits, (40, n)), T.f32_device(xh)):
            st = torch.zeros(1, dtype=torch.int32, device="cuda")
            g = hq.hq_encode_tiles(xd, lattice, n, bps, seed, scale=torch.from_numpy(sc).cuda(),
                                   status=st)
            torch.cuda.synchronize()
            res.append((int(st.item()), g))
        for st_val, _ in res:
            assert st_val == (hq.HQ_ST_OVERFLOW if flagged else 0), label
        (_, gf), (_, gg) = res
        has_coset = codec.coset_bits_per_tile(lattice, n) > 0
        for key in ("idx", "rice_k", "tile_bits") + (("coset",) if has_coset else ()):
            assert torch.equal(gf[key], gg[key]), "%s: fast and generic %s differ" % (label, key)
        keep = np.ones(40, bool)
        keep[9] = not flagged
        sub = {k: (v[keep] if isinstance(v, np.ndarray) and v.shape[:1] == (40,) else v)
               for k, v in ora.items()}
        gc = T.u32(gf["coset"])[keep] if has_coset else None
        _, _, _, ok = T.compare_indices(T.host(gf["idx"])[keep], gc, sub, lattice, n, label)
        assert np.array_equal(T.host(gf["rice_k"])[keep][ok].astype(np.int64), sub["rice_k"][ok])
        assert np.array_equal(T.u32(gf["tile_bits"])[keep][ok].astype(np.int64),
                              sub["tile_bits"][ok])


@pytest.mark.parametrize("lattice,n", [("E8", 128), ("D4", 128), ("A2", 128), ("Z", 128),
                                       ("E8", 256), ("E8", 512)])
def test_fast_decode_scale_range(lattice, n):
    """Fast-kernel decode (tile 128, E8 / tiles 256 and 512) of oracle indices under
    caller scales: bf16-valued scales within 2^-80 .. 2^80, fp32 scales with
    24 significant bits (the product with the Hadamard sums needs more than
    fp32 holds), and bf16 scales from 2^-112 to 2^104 whose outputs leave the
    range of the kernels' fp32 shortcuts; every case against the oracle, bit
    for bit (A2 within its tolerance)."""
    rng = np.random.default_rng(23)
    T = 2100
    x = rng.standard_normal((T, n))
    bits = workloads.f32_to_bf16_bits(x.astype(np.float32))
    ora = codec.encode(workloads.bf16_bits_to_f64(bits), lattice, n, 4.0, rht_seed=6)
    # 32 bf16 scales in range; 2000 fp32 scales (about one output in 2^16
    # would round twice through an fp32 product); 68 bf16 scales at the
    # extremes, the smallest (2^-126 .. 2^-118) giving subnormal outputs that
    # flush to zero
    sc = np.concatenate([codec.bf16_rne(2.0 ** rng.uniform(-80, 80, 32)),
                         (2.0 ** rng.uniform(-40, 40, 2000)).astype(np.float32).astype(np.float64),
                         codec.bf16_rne(2.0 ** rng.uniform(-126, -118, 34)),
                         codec.bf16_rne(2.0 ** rng.uniform(-112, 104, 34))])
    fp32 = sc[32:2032]
    assert np.all(codec.bf16_bits(fp32).astype(np.uint32) << 16 !=
                  fp32.astype(np.float32).view(np.uint32))
    ora["scale"] = sc
    say("case: %s/%d decode, bf16, fp32 and extreme scales" % (lattice, n))
    check_decode(ora, lattice, n, 6, "%s/%d scale range" % (lattice, n), exact=(lattice != "A2"))
    if lattice == "E8" and n >= 256:
        # every other tile with indices up to +-100, whose sum |P| leaves
        # int16 (the fast decoders' fp32 Hadamard), beside ordinary tiles
        big = dict(ora)
        big["idx"] = np.array(ora["idx"], np.int64).reshape(T, n)
        big["idx"][::2] = rng.integers(-100, 101, size=((T + 1) // 2, n))
        big["scale"] = codec.bf16_rne(2.0 ** rng.uniform(-20, 20, T))
        say("case: %s/%d decode, large indices" % (lattice, n))
        check_decode(big, lattice, n, 6, "%s/%d large indices" % (lattice, n))
