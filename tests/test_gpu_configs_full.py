"""Full parity of the lattice sweep matrix and of the dithered KV cache, every
tile against the oracle, in the calls the benchmark times.

* Sweep: one 4096 x 14336 bf16 N(0, 0.02^2) matrix through D4, A2, Z (tile
  128) and E8 (tiles 256 and 512) at 2, 3 and 4 bps (hq_encode_tiles, auto
  scale, RHT seed 1; hq_decode_tiles to bf16).
* KV: K and V [8 heads, 32768 positions, 128] bf16 with per-channel offsets,
  E8 at 4 bps with the subtractive dither (hq_kv_encode, RHT seed 1, dither
  seed 2, K numbered from 0 and V after it; hq_decode_tiles to bf16 with the
  same dither).

The oracle runs over tile chunks in a pool of forked single-threaded
processes; the GPU results are copied to the host before the pool starts.
Per tile and block:
  * scales equal the oracle's (tiles whose fp64 pre-rounding scale sits on a
    bf16 midpoint are counted and skipped);
  * indices and coset bits bit-exact except on oracle near-ties (margin
    < 1e-6), whose count must stay within 1e-5 of the blocks;
  * rice_k and tile_bits exact on tiles whose indices match;
  * the decoded bf16 values equal the oracle's decode of the GPU's own
    indices rounded to bf16 (A2: within 1e-5 Delta plus half a bf16 ulp,
    its sqrt(3) coordinates rounding in fp64 in a different order).
Counts are printed and, when HQ_PARITY_RECORD names a file, appended to it as
one JSON line per case.
"""

import json
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import codec
import hq_testlib as T

pytestmark = pytest.mark.gpu

from lattice_post_quantization_amd import hq  # noqa: E402  (fails loudly if unbuilt)

CHUNK = 4096          # tiles per worker task
_HOST = {}            # the case's inputs and GPU results, inherited by the fork


def _midpoint_close(pre, rel=1e-9):
    m, _ = np.frexp(np.asarray(pre, np.float64))
    t = m * 256.0
    return np.abs(t - np.floor(t) - 0.5) < rel * t


def _check_chunk(task):
    from threadpoolctl import threadpool_limits
    t0, t1 = task
    H = _HOST
    lat, n, bps, seed = H["lattice"], H["n"], H["bps"], H["seed"]
    ds, base = H["dither_seed"], H["dither_base"]
    d = codec.DIM[lat]
    X = workloads.bf16_bits_to_f64(H["bits"][t0:t1])
    with threadpool_limits(limits=1):
        kw = {} if ds is None else {"dither_seed": ds, "dither_base": base + t0}
        ora = codec.encode(X, lat, n, bps, rht_seed=seed, **kw)
        gi = H["idx"][t0:t1].astype(np.int64)
        gc = H["coset"][t0:t1]
        gs = H["scale"][t0:t1].astype(np.float64)
        pre = np.sqrt(np.sum(X * X, axis=1) / n) * codec.scale_constant(lat, bps)
        skip = _midpoint_close(pre)
        r = {"tiles": t1 - t0, "skips": int(skip.sum())}
        r["scale_bad"] = int(np.sum((gs != ora["scale"]) & ~skip))
        keep = gs == ora["scale"]
        bad = np.any(gi[keep].reshape(-1, n // d, d) != ora["idx"][keep].reshape(-1, n // d, d),
                     axis=-1)
        if codec.coset_bits_per_tile(lat, n):
            bad |= (codec.unpack_cosets(gc[keep], lat, n) !=
                    codec.unpack_cosets(ora["coset"][keep], lat, n))
        near = ora["margin"][keep] < T.NEAR_TIE
        r["blocks"] = int(bad.size)
        r["mismatch"] = int(bad.sum())
        r["mismatch_outside_near"] = int(np.sum(bad & ~near))
        r["near_ties"] = int(near.sum())
        ok = ~np.any(bad, axis=1)
        r["rate_bad"] = int(np.sum(H["rice_k"][t0:t1][keep][ok] != ora["rice_k"][keep][ok]) +
                            np.sum(H["tile_bits"][t0:t1][keep][ok] != ora["tile_bits"][keep][ok]))
        # decode of the GPU's own indices and scales
        x = codec.decode(gi, gc, gs, lat, n, seed, **kw)
        y = H["y"][t0:t1]
        if lat == "A2":
            yg = workloads.bf16_bits_to_f64(y)
            tol = 1e-5 * gs[:, None] + 0.5 * np.abs(x) * 2.0 ** -7 + 2.0 ** -126
            r["decode_bad"] = int(np.sum(np.abs(yg - x) > tol))
        else:
            r["decode_bad"] = int(np.sum(y != codec.bf16_bits(codec.bf16_rne(x))))
    return r


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


def _run_case(label, rec_base, bits, g, y, lattice, n, bps, seed, dither_seed=None,
              dither_base=0):
    """Copies the case to the host, runs the oracle comparison over every
    tile in a fork pool, records and asserts the counts."""
    _HOST.clear()
    _HOST.update({
        "lattice": lattice, "n": n, "bps": bps, "seed": seed, "dither_seed": dither_seed,
        "dither_base": dither_base, "bits": bits.reshape(-1, n),
        "scale": T.host(g["scale"]), "idx": T.host(g["idx"]).reshape(-1, n),
        "coset": T.u32(g["coset"]).reshape(bits.size // n, -1),
        "rice_k": T.host(g["rice_k"]).astype(np.int64),
        "tile_bits": T.u32(g["tile_bits"]).astype(np.int64),
        "y": T.bf16_host_bits(y).reshape(-1, n)})
    n_t = _HOST["bits"].shape[0]
    tasks = [(a, min(a + CHUNK, n_t)) for a in range(0, n_t, CHUNK)]
    pool = mp.get_context("fork").Pool(_workers())
    try:
        parts = pool.map(_check_chunk, tasks, chunksize=1)
    finally:
        pool.close()
        pool.join()
        _HOST.clear()
    tot = {k: sum(p[k] for p in parts) for k in parts[0]}
    rec = dict(rec_base)
    rec.update(tot)
    rec.update({"near_tie_fraction": tot["near_ties"] / tot["blocks"],
                "mismatch_fraction": tot["mismatch"] / tot["blocks"]})
    print("  " + json.dumps(rec), flush=True)
    path = os.environ.get("HQ_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    assert tot["tiles"] == n_t, label
    assert tot["scale_bad"] == 0, label
    assert tot["mismatch_outside_near"] == 0, label
    assert tot["mismatch"] <= T.NEAR_TIE_CAP * tot["blocks"], label
    assert tot["rate_bad"] == 0, label
    assert tot["decode_bad"] == 0, label


@pytest.mark.parametrize("lattice,n", [("D4", 128), ("A2", 128), ("Z", 128), ("E8", 256),
                                       ("E8", 512)])
def test_lattice_sweep_full_parity(lattice, n):
    bits = workloads.sweep_matrix()
    rows, cols = bits.shape
    xd = T.bf16_device(bits, (rows, cols))
    for bps in (2.0, 3.0, 4.0):
        label = "sweep %s/%d R=%g, every tile" % (lattice, n, bps)
        print("case: " + label, flush=True)
        g = hq.hq_encode_tiles(xd, lattice, n, bps, 1)
        y = hq.hq_decode_tiles(g["idx"], g["coset"], g["scale"], lattice, n, 1, torch.bfloat16)
        torch.cuda.synchronize()
        _run_case(label, {"workload": "lattice sweep matrix 4096x14336 bf16 N(0, 0.02^2), "
                                      "auto scale, RHT seed 1, bf16 decode",
                          "lattice": lattice, "tile": n, "bps": bps},
                  bits, g, y, lattice, n, bps, 1)
        del g, y


def test_kv_cache_full_parity():
    kb, vb = workloads.kv_layer()
    nvec = kb.shape[0] * kb.shape[1]
    for name, bits, base in (("K", kb, 0), ("V", vb, nvec)):
        label = "kv %s [8, 32768, 128], E8 4 bps dithered, every vector" % name
        print("case: " + label, flush=True)
        xd = T.bf16_device(bits, (nvec, 128))
        g = hq.hq_kv_encode(xd, 4.0, 1, dither_seed=2, dither_base=base)
        y = hq.hq_decode_tiles(g["idx"], g["coset"], g["scale"], "E8", 128, 1, torch.bfloat16,
                               dither_seed=2, dither_base=base)
        torch.cuda.synchronize()
        _run_case(label, {"workload": "KV cache %s [8 heads, 32768, 128] bf16, per-channel "
                                      "offsets on 4 channels, E8 tile 128, 4 bps, subtractive "
                                      "dither (seed 2), RHT seed 1, bf16 decode" % name,
                          "lattice": "E8", "tile": 128, "bps": 4.0},
                  bits, g, y, "E8", 128, 4.0, 1, dither_seed=2, dither_base=base)
        del xd, g, y
