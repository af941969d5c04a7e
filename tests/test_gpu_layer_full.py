"""Full parity of one Llama-3.1-8B-shaped decoder layer (seven bf16
projections, 851968 tiles of 256, outlier columns) at 3, 4 and 5 bps, in the
launch configuration the benchmark times: one batched encode of the seven
matrices (auto scale, RHT seed 0), one batched decode to bf16 and one batched
rate + pack, all through the C ABI.

Every tile is checked.  The oracle runs over tile chunks in a pool of forked
processes (one BLAS thread each); the GPU results are copied to the host
before the pool starts, so the workers read them and nothing crosses back.
Per tile and block:
  * scales equal the oracle's (tiles whose fp64 pre-rounding scale sits on a
    bf16 midpoint are counted and skipped);
  * indices and coset bits bit-exact except on oracle near-ties (margin
    < 1e-6), whose count must stay within 1e-5 of the blocks;
  * the encoder's rice_k and tile_bits exact on tiles whose indices match;
  * the decoded bf16 weights equal the oracle's decode of the GPU's own
    indices, rounded to bf16, bit for bit;
  * the packed stream equals the oracle packer's on the GPU's indices word
    for word, with the same per-tile k, bits and word offsets.
Counts are printed and, when HQ_PARITY_RECORD names a file, appended to it as
one JSON line per rate.
"""

import json
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import codec, rice
import hq_testlib as T

pytestmark = pytest.mark.gpu

from lattice_post_quantization_amd import hq  # noqa: E402  (fails loudly if unbuilt)

N = 256
CHUNK = 4096          # tiles per worker task
_HOST = {}            # host copies of inputs and GPU results, inherited by the fork


def _midpoint_close(pre, rel=1e-9):
    m, _ = np.frexp(np.asarray(pre, np.float64))
    t = m * 256.0
    return np.abs(t - np.floor(t) - 0.5) < rel * t


def _check_chunk(task):
    from threadpoolctl import threadpool_limits
    m, t0, t1, bps = task
    H = _HOST[m]
    X = workloads.bf16_bits_to_f64(H["bits"][t0:t1])
    with threadpool_limits(limits=1):
        ora = codec.encode(X, "E8", N, bps, rht_seed=0)
        gi = H["idx"][t0:t1].astype(np.int64)
        gc = H["coset"][t0:t1]
        gs = H["scale"][t0:t1].astype(np.float64)
        skip = _midpoint_close(np.sqrt(np.sum(X * X, axis=1) / N) * codec.scale_constant("E8", bps))
        r = {"tiles": t1 - t0, "skips": int(skip.sum())}
        r["scale_bad"] = int(np.sum((gs != ora["scale"]) & ~skip))
        keep = gs == ora["scale"]
        # block comparison on the tiles whose scales agree
        gb = gi[keep].reshape(-1, N // 8, 8)
        ob = ora["idx"][keep].reshape(-1, N // 8, 8)
        bad = np.any(gb != ob, axis=-1)
        bad |= codec.unpack_cosets(gc[keep], "E8", N) != codec.unpack_cosets(ora["coset"][keep], "E8", N)
        near = ora["margin"][keep] < T.NEAR_TIE
        r["blocks"] = int(bad.size)
        r["mismatch"] = int(bad.sum())
        r["mismatch_outside_near"] = int(np.sum(bad & ~near))
        r["near_ties"] = int(near.sum())
        ok = ~np.any(bad, axis=1)
        r["enc_rate_bad"] = int(np.sum(H["rice_k"][t0:t1][keep][ok] != ora["rice_k"][keep][ok]) +
                                np.sum(H["tile_bits"][t0:t1][keep][ok] != ora["tile_bits"][keep][ok]))
        # decode of the GPU's own indices and scales
        x = codec.decode(gi, gc, gs, "E8", N, 0)
        want = codec.bf16_bits(codec.bf16_rne(x))
        r["decode_bad"] = int(np.sum(H["y"][t0:t1] != want))
        # rate + pack of the GPU's indices
        k, tb, words, off = rice.pack(gi, gc, 32)
        goff = H["off"][t0:t1 + 1] - H["off"][t0]
        r["pack_rate_bad"] = int(np.sum(H["rk"][t0:t1] != k) + np.sum(H["rb"][t0:t1] != tb))
        r["pack_off_bad"] = int(np.sum(goff != off))
        gw = H["words"][H["off"][t0]:H["off"][t1]]
        r["pack_words_bad"] = int(gw.size != words.size or not np.array_equal(gw, words))
        r["bits"] = int(tb.sum())
    return r


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


@pytest.mark.parametrize("bps", [3.0, 4.0, 5.0])
def test_llama_layer_full_parity(bps):
    print("case: llama layer 0, all seven projections, every tile, R=%g" % bps, flush=True)
    xs, bits = [], []
    for m, (name, rows, cols) in enumerate(workloads.LLAMA_LAYER):
        b = workloads.llama_matrix(m, layer=0)
        bits.append(b.reshape(-1, N))
        xs.append(T.bf16_device(b, (rows, cols)))
    encs = hq.hq_encode_batch(xs, "E8", N, bps, 0)
    ys = hq.hq_decode_batch(encs, "E8", N, 0, torch.bfloat16)
    rates = hq.hq_rate_batch(encs, "E8", N, pack=True)
    given = hq.hq_rate_batch(encs, "E8", N, pack=True, given=True)
    torch.cuda.synchronize()
    for r, g in zip(rates, given):
        nw = int(r["tile_word_offset"][-1])
        assert torch.equal(r["tile_word_offset"], g["tile_word_offset"])
        assert torch.equal(r["stream"][:nw], g["stream"][:nw])
        assert int(r["total_bits"][0]) == int(g["total_bits"][0])
    _HOST.clear()
    for m, (e, y, r) in enumerate(zip(encs, ys, rates)):
        nw = int(r["tile_word_offset"][-1])
        _HOST[m] = {
            "bits": bits[m], "scale": T.host(e["scale"]), "idx": T.host(e["idx"]).reshape(-1, N),
            "coset": T.u32(e["coset"]).reshape(-1, 1), "rice_k": T.host(e["rice_k"]).astype(np.int64),
            "tile_bits": T.u32(e["tile_bits"]).astype(np.int64),
            "y": T.bf16_host_bits(y).reshape(-1, N),
            "rk": T.host(r["rice_k"]).astype(np.int64), "rb": T.u32(r["tile_bits"]).astype(np.int64),
            "off": T.host(r["tile_word_offset"]).astype(np.int64),
            "words": T.u32(r["stream"])[:nw].copy(),
            "total": int(T.host(r["total_bits"])[0]),
        }
    del xs, encs, ys, rates, given
    tasks = [(m, t0, min(t0 + CHUNK, len(_HOST[m]["bits"])), bps)
             for m in range(len(_HOST)) for t0 in range(0, len(_HOST[m]["bits"]), CHUNK)]
    ctx = mp.get_context("fork")
    pool = ctx.Pool(_workers())
    try:
        parts = pool.map(_check_chunk, tasks, chunksize=1)
    finally:
        pool.close()
        pool.join()
    tot = {k: sum(p[k] for p in parts) for k in parts[0]}
    bits_by_matrix = {}
    for (m, _, _, _), p in zip(tasks, parts):
        bits_by_matrix[m] = bits_by_matrix.get(m, 0) + p["bits"]
    rec = dict(tot)
    rec.update({"workload": "llama3.1-8b-shaped layer 0, seven projections (bf16, outlier "
                            "columns), E8 tile 256, auto scale, RHT seed 0",
                "bps": bps, "near_tie_fraction": tot["near_ties"] / tot["blocks"],
                "mismatch_fraction": tot["mismatch"] / tot["blocks"]})
    print("  " + json.dumps(rec), flush=True)
    path = os.environ.get("HQ_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    assert tot["tiles"] == sum(len(h["bits"]) for h in _HOST.values())
    assert tot["scale_bad"] == 0
    assert tot["mismatch_outside_near"] == 0
    assert tot["mismatch"] <= T.NEAR_TIE_CAP * tot["blocks"]
    assert tot["enc_rate_bad"] == 0
    assert tot["decode_bad"] == 0
    assert tot["pack_rate_bad"] == 0 and tot["pack_off_bad"] == 0 and tot["pack_words_bad"] == 0
    for m, h in _HOST.items():
        assert h["total"] == bits_by_matrix[m]
    _HOST.clear()
