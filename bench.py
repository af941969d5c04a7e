#!/usr/bin/env python3
"""E8 encode+decode throughput of the HyperQuant hot path on one MI355X.

Workload: the Llama-3.1-8B-shaped 32-layer stack (per layer q/o 4096x4096,
k/v 1024x4096, gate/up 14336x4096, down 4096x14336; 6.98e9 bf16 weights,
13.96 GB), entries N(0, 0.02^2) with 0.1% of input columns replaced by
10 * Student-t(4) outliers, drawn on the GPU (seed per layer).  One step
streams the whole stack: for each layer, encode its seven matrices (E8,
4 bps, tile 256, auto scale, RHT seed = layer index) with one batched call,
then decode them to bf16 with another.  Inputs and output buffers are
resident in HBM before timing starts.

Prints one JSON line.  value = bf16 GB/s in = 2 * weights / step time.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Algorithmic bytes per 256-weight E8 tile (bf16 in / int8 idx / one coset
# word / uint8 k / uint32 bits / fp32 scale).
ENC_BYTES_PER_TILE = 512 + 256 + 4 + 1 + 4 + 4
DEC_BYTES_PER_TILE = 256 + 4 + 4 + 512

# Measured per kernel (rocprofv3, summarised in profiles/): HBM bytes per
# algorithmic byte (FETCH_SIZE + WRITE_SIZE per dispatch, each scaled by
# what the same counter reads for a copy of known size, over the dispatch's
# algorithmic bytes) and VALU lane-operations (SQ_INSTS_VALU x 64 lanes) per
# algorithmic byte and per weight.  They describe the kernels built from the
# sources with this sha256 and are reported only while the sources match.
KERNEL_SOURCES = ("hq_e8fast.hip", "hq_lanes.h", "hq_device.h", "hq_internal.h")
MEASURED_TRAFFIC = {
    "sources_sha256": "517c6c08f6cdc18e20a475e02dcbfc54f65c7b52939048fedc67442e97b80a4e",
    "encode": {"bytes_per_byte": 1.0041, "valu_lane_ops_per_byte": 9.65298,
               "valu_lane_ops_per_weight": 29.45},
    "decode": {"bytes_per_byte": 1.0011, "valu_lane_ops_per_byte": 3.41564,
               "valu_lane_ops_per_weight": 10.35},
    "codec": {"bytes_per_byte": 1.0037, "valu_lane_ops_per_byte": 7.00113,
              "valu_lane_ops_per_weight": 21.29},
}
# VALU issue roof: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (a wave64 instruction
# occupies a SIMD for 4 cycles; fp64 add / mul / fma issue at the same rate)
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "lattice_post_quantization_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--bps", type=float, default=4.0)
    ap.add_argument("--cpu-baseline", type=int, default=1,
                    help="time the oracle on the 1024x1024 matrix and one whole layer "
                         "(rank 0, N=1), and compare it with the GPU's results")
    ap.add_argument("--pipeline", type=int, default=1,
                    help="also time the pipelined form of the step (one launch encodes layer "
                         "l and decodes layer l - 1) and report it as the headline")
    ap.add_argument("--cold-steps", type=int, default=2,
                    help="also time this many cache-cold steps (all encodes, then all "
                         "decodes; reported beside the headline)")
    ap.add_argument("--secondary", type=int, default=1,
                    help="after the timed steps, also time the pack pass and the KV path "
                         "(reported beside the headline, never in it)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a kernel of "
                         "known traffic that scales the profiler's byte counters)")
    return ap.parse_args()


# ------------------------------------------------------------ CPU baseline
#
# The oracle (fp64 NumPy, unmodified) timed on the host cores on the two
# workloads it finishes in seconds: the 1024x1024 fp32 matrix (E8, 4 bps,
# tile 256, RHT seed 1) and one whole layer of the stack (the benchmarked
# layer 0, copied from the GPU; E8, 4 bps, tile 256, RHT seed 0).  Work:
# encode (rotation, nearest point, strip, Rice k and bits) and decode.  One
# untimed warm-up pass, which also compares the oracle with the GPU's own
# results of the same inputs (the parity record of the line), then three
# timed passes; the median is reported.  Tile chunks are spread over a pool
# of forked single-threaded processes.

_CPU = {}     # inputs and GPU results, set before the pool forks


def _oracle_chunk(task):
    """One chunk of tiles: oracle encode + decode; with compare=True also
    the comparison against the GPU's results of the same tiles."""
    from threadpoolctl import threadpool_limits

    import numpy as np

    from oracle import codec
    key, t0, t1, compare = task
    w = _CPU[key]
    with threadpool_limits(limits=1):
        X = w["x"](t0, t1)
        e = codec.encode(X, "E8", 256, w["bps"], rht_seed=w["seed"])
        codec.decode(e["idx"], e["coset"], e["scale"], "E8", 256, w["seed"])
        if not compare:
            return None
        g = w["gpu"]
        gs = g["scale"][t0:t1].astype(np.float64)
        keep = gs == e["scale"]
        gi = g["idx"][t0:t1].astype(np.int64)
        bad = np.any((gi[keep] != e["idx"][keep]).reshape(-1, 32, 8), axis=-1)
        gc = codec.unpack_cosets(g["coset"][t0:t1][keep], "E8", 256)
        bad |= gc != codec.unpack_cosets(e["coset"][keep], "E8", 256)
        near = e["margin"][keep] < 1e-6
        ok = ~np.any(bad, axis=1)
        # decoded weights: the oracle's decode of the GPU's own indices
        yd = codec.bf16_bits(codec.bf16_rne(codec.decode(gi, g["coset"][t0:t1], gs, "E8", 256,
                                                         w["seed"])))
        return {"tiles": t1 - t0, "scale_differs": int(np.sum(~keep)),
                "blocks": int(bad.size), "mismatches": int(bad.sum()),
                "mismatches_outside_near_ties": int(np.sum(bad & ~near)),
                "near_ties": int(near.sum()),
                "rate_differs": int(np.sum(g["rice_k"][t0:t1][keep][ok] != e["rice_k"][keep][ok]) +
                                    np.sum(g["tile_bits"][t0:t1][keep][ok] != e["tile_bits"][keep][ok])),
                "decode_bf16_differs": int(np.sum(g["y"][t0:t1] != yd))}


def cpu_baseline(layer0_host, small_host, bps, runs=3):
    """Times the oracle on the host cores (see above); returns (cpu_baseline
    object, parity record)."""
    import multiprocessing as mp
    import statistics

    import numpy as np

    import workloads
    from oracle import codec

    _CPU.clear()
    _CPU["small"] = {"x": lambda a, b: codec.tiles(small_host["x"], 256)[a:b], "bps": bps,
                     "seed": 1, "gpu": small_host, "tiles": small_host["x"].size // 256}
    lb = layer0_host["bits"]
    _CPU["layer"] = {"x": lambda a, b: workloads.bf16_bits_to_f64(lb[a:b]), "bps": bps,
                     "seed": 0, "gpu": layer0_host, "tiles": len(lb)}
    host_cpus = os.cpu_count() or 1
    procs = min(host_cpus, 16)          # the CPU share of one GPU on the box
    ctx = mp.get_context("fork")
    pool = ctx.Pool(procs)
    out, parity = {}, {}
    try:
        for key, chunk in (("small", 256), ("layer", 4096)):
            n_t = _CPU[key]["tiles"]
            tasks = [(key, a, min(a + chunk, n_t)) for a in range(0, n_t, chunk)]
            parts = pool.map(_oracle_chunk, [t + (True,) for t in tasks], chunksize=1)
            rec = {k: sum(p[k] for p in parts) for k in parts[0]}
            rec["near_tie_fraction"] = rec["near_ties"] / max(rec["blocks"], 1)
            rec["mismatch_fraction"] = rec["mismatches"] / max(rec["blocks"], 1)
            parity[key] = rec
            walls = []
            for _ in range(runs):
                t0 = time.perf_counter()
                pool.map(_oracle_chunk, [t + (False,) for t in tasks], chunksize=1)
                walls.append(time.perf_counter() - t0)
            print("cpu baseline %s: %s s" % (key, ", ".join("%.2f" % w for w in walls)),
                  file=sys.stderr, flush=True)
            out[key] = (statistics.median(walls), n_t * 256)
    finally:
        pool.close()
        pool.join()
        _CPU.clear()
    wall, n_w = out["layer"]
    base = {
        "value": round(2.0 * n_w / wall / 1e9, 6),
        "unit": "GB/s (bf16 in)",
        "cores": procs,
        "host_cpu_count": host_cpus,
        "kind": "oracle",
        "sample": "one whole layer of the stack (layer 0, %d weights, copied from the GPU), "
                  "E8 4 bps tile 256, oracle encode (rotation, nearest point with margins, "
                  "strip, Rice k and bits) + decode; median of %d passes after a warm-up, "
                  "%.2f s; %d single-threaded processes on a host reporting %d CPUs"
                  % (n_w, runs, wall, procs, host_cpus),
        "small_fp32_1024x1024": {"median_s": round(out["small"][0], 4),
                                 "gbs_in": round(4.0 * out["small"][1] / out["small"][0] / 1e9, 6)},
    }
    return base, parity


# ------------------------------------------------------------------- GPU

def rate_and_quality(layer, bps):
    """Itemized rate of the benchmarked layer 0 (all seven matrices) from
    the GPU's rate pass (the encoder's k and bits given), and the
    reconstruction error of its bf16 decode (outside the timed region).
    Items (bits): the Rice payload, one coset bit per E8 block, the 4-bit k
    field, the word padding of the packed stream, and the per-tile scale --
    16 bits as a bf16 value (lossless for the auto scale) or 32 as the
    checkpoint file stores it, with its 64-bit tile word offsets."""
    import torch

    from lattice_post_quantization_amd import hq
    xs, encs, ys = layer
    rates = hq.hq_rate_batch(encs, "E8", 256, pack=True, given=True)
    tb = torch.cat([r["tile_bits"].view(torch.int32).to(torch.int64) for r in rates])
    words = sum(int(r["tile_word_offset"][-1]) for r in rates)
    tiles = int(tb.numel())
    w = tiles * 256
    coset, kf = 32 * tiles, 4 * tiles
    payload = int(tb.sum()) - coset - kf
    pad = 32 * words - int(tb.sum())
    stream = payload + coset + kf + pad
    minimal = stream + 16 * tiles
    stored = stream + 32 * tiles + 64 * (tiles + len(rates))
    num = den = err_g = 0.0
    g_e8 = 929.0 / 12960.0
    for x, e, y in zip(xs, encs, ys):
        xd = x.double().view(-1, 256)
        d = y.double().view(-1, 256) - xd
        num += float((d * d).sum())
        den += float((xd * xd).sum())
        sc = e["scale"].double().view(-1, 1)
        err_g += float(((d * d) / (g_e8 * sc * sc)).sum())
    torch.cuda.synchronize()
    return {
        "workload": "layer 0 of the stack (seven matrices, %d weights), E8 %g bps, tile 256" % (w, bps),
        "bits": {"payload": payload, "coset": coset, "k_field": kf, "padding": pad,
                 "scale_bf16": 16 * tiles, "scale_fp32_as_stored": 32 * tiles,
                 "offsets_as_stored": 64 * (tiles + len(rates))},
        "bits_per_weight": {"payload": round(payload / w, 4), "stream": round(stream / w, 4),
                            "with_bf16_scale": round(minimal / w, 4),
                            "as_stored": round(stored / w, 4)},
        "compression_vs_bf16": {"with_bf16_scale": round(16.0 * w / minimal, 3),
                                "as_stored": round(16.0 * w / stored, 3)},
        "relative_mse": num / den,
        "sqnr_db": round(-10.0 * math.log10(num / den), 3),
        "mse_over_G_delta2": round(err_g / w, 4),
    }


def time_calls(fn, reps, warm=2):
    """Average milliseconds of fn() over reps calls, HIP events on the
    current stream (fn launches on it)."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def kv_per_vector(kcache, bps, dev, n_vec=64, n_seeds=1024):
    """Per-vector bias of the reconstruction, dither against rotation-only:
    n_vec fixed K vectors (every 4096th of the cache) through encode and
    fp32 decode under n_seeds dither seeds.  With the dither the error is
    uniform on the E8 cell scaled by Delta: z = mean error / (Delta
    sqrt(G / S)) is standard per coordinate and MSE / (G Delta^2) = 1;
    rotation-only errors stay fixed, so their z grows as sqrt(S)."""
    import torch

    from lattice_post_quantization_amd import hq

    g_e8 = 929.0 / 12960.0            # normalized second moment of E8 (Conway-Sloane)
    xd = kcache[torch.arange(n_vec, device=dev) * 4096].contiguous()
    x = xd.double()
    o = hq.hq_kv_encode(xd, bps, 1, dither_seed=1)
    delta = o["scale"].double()[:, None]
    y = torch.empty(xd.shape, dtype=torch.float32, device=dev)
    acc = torch.zeros_like(x)
    acc2 = torch.zeros_like(x)
    for s in range(1, n_seeds + 1):
        hq.hq_kv_encode(xd, bps, 1, dither_seed=s, out=o)
        hq.hq_decode_tiles(o["idx"], o["coset"], o["scale"], "E8", 128, 1, torch.float32,
                           dither_seed=s, out=y)
        e = y.double() - x
        acc += e
        acc2 += e * e
    unit = delta * math.sqrt(g_e8 / n_seeds)
    z = acc / n_seeds / unit
    o0 = hq.hq_kv_encode(xd, bps, 1)
    e0 = hq.hq_decode_tiles(o0["idx"], o0["coset"], o0["scale"], "E8", 128, 1,
                            torch.float32).double() - x
    z0 = e0 / unit
    return {"workload": "%d K vectors (every 4096th of the cache), %d dither seeds, fp32 decode; "
                        "z = per-coordinate mean error over the seeds / (Delta sqrt(G(E8) / S))"
                        % (n_vec, n_seeds),
            "dither": {"z_rms": round(float(torch.sqrt((z * z).mean())), 4),
                       "z2_per_vector_max": round(float((z * z).mean(1).max()), 4),
                       "mse_over_G_delta2": round(float((acc2 / n_seeds / (g_e8 * delta * delta)).mean()), 4)},
            "rotation_only": {"z_rms": round(float(torch.sqrt((z0 * z0).mean())), 2),
                              "z_rms_per_vector_min": round(float(torch.sqrt((z0 * z0).mean(1)).min()), 2),
                              "mse_over_G_delta2": round(float((e0 * e0 / (g_e8 * delta * delta)).mean()), 4)}}


def secondary(layer0, bps, dev):
    """Steps outside the headline: the rate + pack pass over one layer's
    indices (its own pass over the encoder's output), the stream decoder on
    the result, GEMV from the indices, the variants (rate control, tile
    512), the lattice sweep matrix through every lattice, and the KV path
    (dithered E8 encode and decode of one layer's K and V cache,
    [8, 32768, 128] each)."""
    import numpy as np
    import torch

    import workloads
    from lattice_post_quantization_amd import hq
    _, encs, _ = layer0
    outs = [hq.hq_rate(e["idx"], e["coset"], "E8", 256, pack=True) for e in encs]

    def pack_layer():
        for e, o in zip(encs, outs):
            hq.hq_rate(e["idx"], e["coset"], "E8", 256, pack=True, out=o)

    ms = time_calls(pack_layer, 10)
    torch.cuda.synchronize()
    tiles = sum(e["idx"].numel() for e in encs) // 256
    words = sum(int(o["tile_word_offset"][-1].item()) for o in outs)
    # the method reads idx + coset once and writes k, bits, offsets and the
    # words (this implementation reads the indices twice: rate, then pack)
    alg = tiles * (256 + 4) + tiles * (1 + 4 + 8) + 4 * words
    # the same packing with the encoder's rice_k and tile_bits (HQ_RATE_GIVEN):
    # reads idx + coset + k + bits once, writes the offsets and the words
    outs_g = [hq.hq_rate(e["idx"], e["coset"], "E8", 256, pack=True, given=e) for e in encs]

    def pack_layer_given():
        for e, o in zip(encs, outs_g):
            hq.hq_rate(e["idx"], e["coset"], "E8", 256, pack=True, out=o, given=e)

    ms_gv = time_calls(pack_layer_given, 10)
    torch.cuda.synchronize()
    same_g = all(torch.equal(a["stream"][:int(a["tile_word_offset"][-1])],
                             b["stream"][:int(b["tile_word_offset"][-1])])
                 for a, b in zip(outs, outs_g))
    alg_g = tiles * (256 + 4 + 1 + 4) + tiles * 8 + 4 * words
    # both in one batched call for the layer
    wsr = torch.empty(max(16, sum(hq.rate_workspace_bytes(e["idx"].numel() // 256)
                                  for e in encs)), dtype=torch.uint8, device=dev)
    outs_b = hq.hq_rate_batch(encs, "E8", 256, pack=True, workspace=wsr)
    outs_bg = hq.hq_rate_batch(encs, "E8", 256, pack=True, given=True, workspace=wsr)
    ms_b = time_calls(lambda: hq.hq_rate_batch(encs, "E8", 256, pack=True, workspace=wsr,
                                               outs=outs_b), 10)
    ms_bg = time_calls(lambda: hq.hq_rate_batch(encs, "E8", 256, pack=True, given=True,
                                                workspace=wsr, outs=outs_bg), 10)
    torch.cuda.synchronize()
    same_b = all(torch.equal(a["stream"][:int(a["tile_word_offset"][-1])],
                             b["stream"][:int(b["tile_word_offset"][-1])])
                 for a, b in zip(outs, outs_b))
    pack = {"workload": "rate + pack of one Llama-3.1-8B-shaped layer's E8 indices "
                        "(seven calls, %d tiles; and one batched call)" % tiles,
            "us": round(ms * 1e3, 2), "algorithmic_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
            "us_batched": round(ms_b * 1e3, 2),
            "us_batched_encoder_rate_given": round(ms_bg * 1e3, 2),
            "batched_stream_identical": bool(same_b),
            "us_encoder_rate_given": round(ms_gv * 1e3, 2),
            "given_algorithmic_gbs": round(alg_g / (ms_gv * 1e-3) / 1e9, 1),
            "given_stream_identical": bool(same_g),
            "stream_bits_per_weight": round(32.0 * words / (tiles * 256), 4)}

    # the stream decoder on the same streams (the first calls check the
    # offsets against the streams; the timed ones skip that read-back)
    unp = [hq.hq_unpack(o["stream"], o["tile_word_offset"], "E8", 256) for o in outs]

    def unpack_layer():
        for o, u in zip(outs, unp):
            hq.hq_unpack(o["stream"], o["tile_word_offset"], "E8", 256, out=u, trusted=True)

    ms_u = time_calls(unpack_layer, 10)
    torch.cuda.synchronize()
    same = all(torch.equal(u["idx"].view(-1), e["idx"].view(-1)) for u, e in zip(unp, encs))
    # the seven streams in one call (one lane per tile: together they fill the GPU)
    unp_b = hq.hq_unpack_batch(outs, "E8", 256)

    def unpack_layer_batched():
        hq.hq_unpack_batch(outs, "E8", 256, outs=unp_b, trusted=True)

    ms_ub = time_calls(unpack_layer_batched, 10)
    torch.cuda.synchronize()
    same_b = all(torch.equal(u["idx"].view(-1), e["idx"].view(-1)) for u, e in zip(unp_b, encs))
    # reads the words and offsets, writes idx, coset and k
    alg_u = 4 * words + 8 * (tiles + len(encs)) + tiles * (256 + 4 + 1)
    unpack = {"workload": "Rice stream decode of the same layer's packed streams: one batched "
                          "call (seven matrices), beside seven single calls",
              "us": round(ms_ub * 1e3, 2), "us_seven_calls": round(ms_u * 1e3, 2),
              "algorithmic_gbs": round(alg_u / (ms_ub * 1e-3) / 1e9, 1),
              "round_trip_exact": bool(same and same_b)}

    # y = W x from the stored indices (m = 1) against a bf16 GEMV of the
    # decoded weights (the same layer's seven matrices)
    _, _, ys = layer0
    xv = [torch.randn(e["idx"].shape[1], device=dev) for e in encs]
    yv = [torch.empty(e["idx"].shape[0], device=dev) for e in encs]
    wsp = [torch.empty(hq.lib().hq_gemv_workspace_bytes(e["idx"].shape[0], e["idx"].shape[1], 1),
                       dtype=torch.uint8, device=dev) for e in encs]

    def gemv_layer():
        for e, x, y, w in zip(encs, xv, yv, wsp):
            hq.hq_gemv(e["idx"], e["coset"], e["scale"], x, rht_seed=0, out=y.view(1, -1),
                       workspace=w)

    xb = [x.to(torch.bfloat16) for x in xv]

    def bf16_layer():
        for wm, x in zip(ys, xb):
            torch.mv(wm, x)

    yv2 = [y.view(1, -1) for y in yv]

    def gemv_layer_batched():
        hq.hq_gemv_batch(encs, xv, rht_seed=0, outs=yv2, workspace=wsb)

    wsb = torch.empty(max(16, sum(int(w.numel()) for w in wsp)), dtype=torch.uint8, device=dev)
    ms_g1 = time_calls(gemv_layer, 10)
    ms_g = time_calls(gemv_layer_batched, 10)
    ms_b = time_calls(bf16_layer, 10)
    rows_cols = [tuple(e["idx"].shape) for e in encs]
    w_total = sum(r * c for r, c in rows_cols)
    alg_g = w_total * (1 + 8 / 256) + sum(4 * (r + c) for r, c in rows_cols)
    gemv = {"workload": "y = W x (one vector, fp32) for the same layer's seven matrices, "
                        "from the E8 indices, one batched call; beside torch.mv on the "
                        "decoded bf16 weights",
            "us": round(ms_g * 1e3, 2), "us_seven_calls": round(ms_g1 * 1e3, 2),
            "bf16_gemv_us": round(ms_b * 1e3, 2),
            "speedup_vs_bf16": round(ms_b / ms_g, 3),
            "algorithmic_gbs": round(alg_g / (ms_g * 1e-3) / 1e9, 1)}

    # Y = W X^T for many vectors on the matrix cores, one batched call for
    # the layer, beside torch.matmul on the decoded bf16 weights
    gemm = {"workload": "Y = W X^T (m fp32 vectors) for the same layer's seven matrices, from "
                        "the E8 indices, one batched call; beside torch.matmul of bf16 X on "
                        "the decoded bf16 weights",
            "by_m": {}}
    for m in (32, 128, 256):
        xm = [torch.randn(m, e["idx"].shape[1], device=dev) for e in encs]
        ym = [torch.empty(m, e["idx"].shape[0], device=dev) for e in encs]
        items = (hq.GemvItem * len(encs))()
        for i, (e, x, y) in enumerate(zip(encs, xm, ym)):
            items[i] = hq.GemvItem(e["idx"].data_ptr(), e["coset"].data_ptr(),
                                   e["scale"].data_ptr(), e["idx"].shape[0], e["idx"].shape[1],
                                   x.data_ptr(), y.data_ptr())
        wsg = torch.empty(max(16, hq.lib().hq_gemm_batch_workspace_bytes(len(encs), items, m)),
                          dtype=torch.uint8, device=dev)

        def gemm_layer():
            hq.hq_gemm_batch(encs, xm, rht_seed=0, outs=ym, workspace=wsg)

        xmb = [x.to(torch.bfloat16) for x in xm]

        def bf16_gemm_layer():
            for wm, x in zip(ys, xmb):
                torch.matmul(x, wm.t())

        ms_m = time_calls(gemm_layer, 10)
        ms_t = time_calls(bf16_gemm_layer, 10)
        gemm["by_m"][str(m)] = {"us": round(ms_m * 1e3, 2), "bf16_matmul_us": round(ms_t * 1e3, 2),
                                "speedup_vs_bf16": round(ms_t / ms_m, 3),
                                "tflops": round(2.0 * m * w_total / (ms_m * 1e-3) / 1e12, 2)}

    # variants on the same layer's weights: per-tile rate control (a bisection
    # over each tile's bf16 scale patterns) and tile 512
    xs0, _, _ = layer0
    rc = [hq.hq_encode_tiles(x, "E8", 256, bps, 0, rate_control=True) for x in xs0]

    def rc_layer():
        for x, o in zip(xs0, rc):
            hq.hq_encode_tiles(x, "E8", 256, bps, 0, rate_control=True, out=o)

    ms_rc = time_calls(rc_layer, 3)
    torch.cuda.synchronize()
    n_w = sum(x.numel() for x in xs0)
    rc_bits = sum(float(o["tile_bits"].double().sum().item()) for o in rc) / n_w
    e512 = [hq.hq_encode_tiles(x, "E8", 512, bps, 0) for x in xs0]
    y512 = [torch.empty_like(x) for x in xs0]

    def enc512():
        for x, o in zip(xs0, e512):
            hq.hq_encode_tiles(x, "E8", 512, bps, 0, out=o)

    def dec512():
        for o, y in zip(e512, y512):
            hq.hq_decode_tiles(o["idx"], o["coset"], o["scale"], "E8", 512, 0, torch.bfloat16,
                               out=y)

    ms_e512, ms_d512 = time_calls(enc512, 5), time_calls(dec512, 5)
    variants = {
        "workload": "the same layer's seven matrices (bf16): per-tile rate control (fast E8 "
                    "kernel), tile 512 (fast E8 kernels)",
        "rate_control_encode_us": round(ms_rc * 1e3, 1),
        "rate_control_bits_per_weight": round(rc_bits, 4),
        "tile512_encode_us": round(ms_e512 * 1e3, 1), "tile512_decode_us": round(ms_d512 * 1e3, 1),
        "tile512_encode_gbs_bf16_in": round(2 * n_w / (ms_e512 * 1e-3) / 1e9, 1)}

    # the lattice sweep matrix (4096 x 14336 bf16 N(0, 0.02^2)): D4, A2 and Z
    # at tile 128 and E8 at tiles 128 and 256, encode and decode at this rate
    sw = workloads.sweep_matrix()
    xs = torch.from_numpy(sw.view(np.int16)).to(dev).view(torch.bfloat16)
    ys = torch.empty_like(xs)
    sweep = {"workload": "one 4096x14336 bf16 N(0, 0.02^2) matrix (%d weights), %g bps, "
                         "bf16 out" % (xs.numel(), bps)}
    for lat, n in (("D4", 128), ("A2", 128), ("Z", 128), ("E8", 128), ("E8", 256)):
        o = hq.hq_encode_tiles(xs, lat, n, bps, 1)
        ms_se = time_calls(lambda: hq.hq_encode_tiles(xs, lat, n, bps, 1, out=o), 10)
        ms_sd = time_calls(lambda: hq.hq_decode_tiles(o["idx"], o["coset"], o["scale"], lat, n,
                                                      1, torch.bfloat16, out=ys), 10)
        sweep["%s_%d" % (lat, n)] = {
            "encode_us": round(ms_se * 1e3, 1), "decode_us": round(ms_sd * 1e3, 1),
            "encode_gbs_bf16_in": round(2 * xs.numel() / (ms_se * 1e-3) / 1e9, 1)}
    del xs, ys

    kb, vb = workloads.kv_layer()
    kvs = [torch.from_numpy(a.reshape(-1, 128).view(np.int16)).to(dev).view(torch.bfloat16)
           for a in (kb, vb)]
    n_vec = sum(t.shape[0] for t in kvs)
    encs_kv = [hq.hq_kv_encode(t, bps, 1, dither_seed=2) for t in kvs]
    ys = [torch.empty_like(t) for t in kvs]

    def kv_enc():
        for t, o in zip(kvs, encs_kv):
            hq.hq_kv_encode(t, bps, 1, dither_seed=2, out=o)

    def kv_dec():
        for o, y in zip(encs_kv, ys):
            hq.hq_decode_tiles(o["idx"], o["coset"], o["scale"], "E8", 128, 1, torch.bfloat16,
                               dither_seed=2, out=y)

    ms_e = time_calls(kv_enc, 10)
    ms_d = time_calls(kv_dec, 10)
    # scores of 64 queries (shared by the heads) against all 8 x 32768
    # compressed keys of the K cache in one call (dither index = key row)
    nq, heads, seq = 64, 8, kb.shape[1]
    qv = torch.randn(nq, 128, device=dev)
    sc = torch.empty(nq, heads * seq, device=dev)
    wsq = torch.empty(hq.lib().hq_kv_scores_workspace_bytes(nq), dtype=torch.uint8, device=dev)

    def kv_scores():
        hq.hq_kv_scores(qv, encs_kv[0], 1, dither_seed=2, dither_base=0, out=sc, workspace=wsq)

    ms_s = time_calls(kv_scores, 10)
    # decode attention: 4 queries per KV head (grouped queries) over each of
    # the 8 heads' compressed K and V, one call per head; beside torch's
    # scaled_dot_product_attention on the decoded bf16 caches
    qa = torch.randn(heads, 4, 128, device=dev)
    oa = torch.empty(heads, 4, 128, device=dev)
    wsa = torch.empty(hq.lib().hq_kv_attention_workspace_bytes(heads, 4, seq), dtype=torch.uint8,
                      device=dev)
    cache = dict(rht_seed=1, dither_seed=2, dither_base=0)

    def kv_attention():
        hq.hq_kv_attention(qa, encs_kv[0], encs_kv[1], k_cache=cache, v_cache=cache, out=oa,
                           workspace=wsa)

    kd = ys[0].view(heads, seq, 128)
    vd = ys[1].view(heads, seq, 128)
    qab = qa.to(torch.bfloat16)

    def bf16_attention():
        torch.nn.functional.scaled_dot_product_attention(qab, kd, vd)

    ms_a = time_calls(kv_attention, 10)
    ms_ab = time_calls(bf16_attention, 10)
    # the same attention on rotation-only caches (no dither to regenerate)
    encs_rot = [hq.hq_kv_encode(t, bps, 1) for t in kvs]
    rot_cache = dict(rht_seed=1)

    def kv_attention_rot():
        hq.hq_kv_attention(qa, encs_rot[0], encs_rot[1], k_cache=rot_cache, v_cache=rot_cache,
                           out=oa, workspace=wsa)

    ms_ar = time_calls(kv_attention_rot, 10)
    del encs_rot
    # per 128-vector: 256 B in / 128 B idx + 4 coset + 1 k + 4 bits + 4 scale
    kv = {"workload": "dithered E8 encode and decode of K and V [8, 32768, 128] bf16 "
                      "(%d vectors of 128, 4 bps)" % n_vec,
          "encode_us": round(ms_e * 1e3, 2), "decode_us": round(ms_d * 1e3, 2),
          "encode_algorithmic_gbs": round(n_vec * (256 + 141) / (ms_e * 1e-3) / 1e9, 1),
          "decode_algorithmic_gbs": round(n_vec * (128 + 8 + 256) / (ms_d * 1e-3) / 1e9, 1),
          "scores_workload": "%d queries against all %d x %d compressed keys of the K cache, "
                             "one call (dither regenerated per key)" % (nq, heads, seq),
          "scores_us": round(ms_s * 1e3, 2),
          "scores_gflops": round(2.0 * nq * heads * seq * 128 / (ms_s * 1e-3) / 1e9, 1),
          "attention_workload": "decode attention of 4 queries per head over all %d heads x %d "
                                "compressed K and V vectors (one call), beside "
                                "scaled_dot_product_attention on the decoded bf16 caches"
                                % (heads, seq),
          "attention_us": round(ms_a * 1e3, 2),
          "attention_rotation_only_us": round(ms_ar * 1e3, 2),
          "attention_bf16_sdpa_us": round(ms_ab * 1e3, 2),
          "attention_cache_gbs": round(2 * heads * seq * (128 + 8) / (ms_a * 1e-3) / 1e9, 1)}
    # bias of the cached inner products at this scale, dither against the
    # rotation-only control: per query q_j, b_j = q_j . mean over the cache
    # of (khat - k), as a z-score against its spread under independent errors
    qb = torch.from_numpy(workloads.kv_queries().astype(np.float32)).to(dev).double()
    bias = {"workload": "K cache [8, 32768, 128] at 4 bps, 4096 queries: z_j = q_j . mean(khat - k) "
                        "/ its standard error; mean and max |z| over the queries"}
    for mode, ds in (("dither", 2), ("rotation_only", None)):
        ek = hq.hq_kv_encode(kvs[0], bps, 1, dither_seed=ds)
        kh = hq.hq_decode_tiles(ek["idx"], ek["coset"], ek["scale"], "E8", 128, 1, torch.float32,
                                dither_seed=ds)
        err = kh.double() - kvs[0].double()
        b = qb @ err.mean(0)
        sd = torch.sqrt((qb * qb) @ (err.var(0) / err.shape[0]))
        z = (b / sd).abs()
        bias[mode] = {"z_mean": round(float(z.mean()), 3), "z_max": round(float(z.max()), 3)}
        del ek, kh, err
    kv["bias"] = bias
    kv["per_vector"] = kv_per_vector(kvs[0], bps, dev)
    return {"pack": pack, "unpack": unpack, "gemv": gemv, "gemm": gemm, "kv": kv,
            "variants": variants,
            "lattice_sweep": sweep}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (tiles are "
              "independent, so a stack shards by layer or row block with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    from lattice_post_quantization_amd import hq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = []
    for layer in range(args.layers):
        xs = [workloads.llama_stack_torch(layer, m, dev) for m in range(len(workloads.LLAMA_LAYER))]
        encs = hq.hq_encode_batch(xs, "E8", 256, args.bps, layer)       # output buffers
        ys = [torch.empty_like(x) for x in xs]
        layers.append((xs, encs, ys))
    torch.cuda.synchronize()
    n_weights = sum(x.numel() for xs, _, _ in layers for x in xs)
    n_tiles = n_weights // 256
    tiles_per_layer = [sum(x.numel() for x in xs) // 256 for xs, _, _ in layers]

    if args.copy_ref_mib > 0:
        src = torch.ones(args.copy_ref_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    L = len(layers)

    class Launches:
        """HIP events recorded around each launch of one kind, on the current
        stream (every call of the library enqueues on it), created up front
        so that no host call sits between launches of the timed region."""

        def __init__(self, n):
            self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            self.k = 0
            self.bytes = []

        def begin(self):
            self.ev[self.k].record()

        def end(self, nbytes):
            self.ev[self.k + 1].record()
            self.k += 2
            self.bytes.append(nbytes)

        def stats(self, steps):
            durs = [self.ev[2 * i].elapsed_time(self.ev[2 * i + 1]) for i in range(self.k // 2)]
            tot_ms = sum(durs)
            return {"launches": len(durs), "avg_us": 1e3 * tot_ms / len(durs),
                    "sum_ms_per_step": tot_ms / steps,
                    "bytes_per_launch": sum(self.bytes) / len(self.bytes),
                    "gbs": sum(self.bytes) / (tot_ms * 1e-3) / 1e9}

    enc_bytes = [t * ENC_BYTES_PER_TILE for t in tiles_per_layer]
    dec_bytes = [t * DEC_BYTES_PER_TILE for t in tiles_per_layer]

    def step_sequential(timers):
        # one launch encodes a layer's seven projections, one launch decodes them
        for layer, (xs, encs, ys) in enumerate(layers):
            if timers:
                timers["encode"].begin()
            hq.hq_encode_batch(xs, "E8", 256, args.bps, layer, outs=encs)
            if timers:
                timers["encode"].end(enc_bytes[layer])
                timers["decode"].begin()
            hq.hq_decode_batch(encs, "E8", 256, layer, torch.bfloat16, outs=ys)
            if timers:
                timers["decode"].end(dec_bytes[layer])

    def step_pipelined(timers):
        # launch l encodes layer l and decodes layer l - 1 (L + 1 launches)
        for layer in range(L + 1):
            xs, encs, _ = layers[layer] if layer < L else ([], None, None)
            dsrc, ys = (layers[layer - 1][1], layers[layer - 1][2]) if layer > 0 else ([], None)
            if timers:
                timers["codec"].begin()
            hq.hq_encode_decode_batch(xs, dsrc, "E8", 256, args.bps, enc_seed=layer,
                                      dec_seed=layer - 1, enc_outs=encs, dec_outs=ys)
            if timers:
                timers["codec"].end((enc_bytes[layer] if layer < L else 0) +
                                    (dec_bytes[layer - 1] if layer > 0 else 0))

    def run(step, kinds):
        for _ in range(args.warmup):
            step(None)
        torch.cuda.synchronize()
        timers = {k: Launches(args.steps * (L + 1)) for k in kinds}
        # timed region: whole steps, bracketed by synchronisation
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        t_start.record()
        for _ in range(args.steps):
            step(timers)
        t_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        gpu_ms = t_start.elapsed_time(t_end)
        return {"ms_per_step": max(gpu_ms, wall * 1e3) / args.steps,
                "host_wall_ms_per_step": wall * 1e3 / args.steps,
                "gpu_event_ms_per_step": gpu_ms / args.steps,
                "kernels": {k: t.stats(args.steps) for k, t in timers.items()}}

    def progress(msg):
        print("bench: " + msg, file=sys.stderr, flush=True)

    progress("inputs ready, timing the sequential step")
    seq = run(step_sequential, ("encode", "decode"))
    progress("timing the pipelined step")
    ref_y = [layers[i][2][m].clone() for i in (0, L - 1) for m in (0, 6)]
    pipe = run(step_pipelined, ("codec",)) if args.pipeline else None
    same = None
    if pipe is not None:
        got = [layers[i][2][m] for i in (0, L - 1) for m in (0, 6)]
        same = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(ref_y, got))
    del ref_y
    head = pipe if pipe is not None else seq
    ms_per_step = head["ms_per_step"]
    kern = dict(seq["kernels"])
    if pipe is not None:
        kern.update(pipe["kernels"])
    dom_name = max(head["kernels"], key=lambda k: head["kernels"][k]["sum_ms_per_step"])
    dominant = kern[dom_name]
    traffic = alu = None
    meas = MEASURED_TRAFFIC.get(dom_name)
    if isinstance(meas, dict) and kernel_sources_sha256() == MEASURED_TRAFFIC["sources_sha256"]:
        # measured HBM bytes per launch: per-tile figures times the tiles of an average launch
        traffic = round(meas["bytes_per_byte"] * dominant["bytes_per_launch"])
        ops = meas["valu_lane_ops_per_byte"] * dominant["bytes_per_launch"]
        achieved = ops / (dominant["avg_us"] * 1e-6)
        alu = {"achieved": round(achieved / 1e12, 2), "peak": round(VALU_PEAK_LANE_OPS / 1e12, 2),
               "unit": "T VALU lane-ops/s (issued)", "frac": round(achieved / VALU_PEAK_LANE_OPS, 4),
               "lane_ops_per_weight": meas["valu_lane_ops_per_weight"]}

    # cache-cold form of the same work: every layer's encode, then every
    # layer's decode, so no decode finds its indices in the 256 MB Infinity
    # Cache (the headline decodes each layer right after its encode)
    cold = None
    if args.cold_steps > 0:
        progress("cache-cold steps")

        def cold_step():
            for layer, (xs, encs, ys) in enumerate(layers):
                hq.hq_encode_batch(xs, "E8", 256, args.bps, layer, outs=encs)
            for layer, (xs, encs, ys) in enumerate(layers):
                hq.hq_decode_batch(encs, "E8", 256, layer, torch.bfloat16, outs=ys)
        cold_step()
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(args.cold_steps):
            cold_step()
        c1.record()
        torch.cuda.synchronize()
        cms = c0.elapsed_time(c1) / args.cold_steps
        cold = {"workload": "the same stack, all 32 encodes then all 32 decodes per step",
                "steps": args.cold_steps, "ms_per_step": round(cms, 4),
                "value": round(2.0 * n_weights / (cms * 1e-3) / 1e9, 3),
                "pct_hbm_peak_algorithmic": round(100.0 * (ENC_BYTES_PER_TILE + DEC_BYTES_PER_TILE)
                                                  * n_tiles / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)}

    # the achievable-bandwidth reference: a plain device copy of 4 GiB
    src = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = time_calls(lambda: dst.copy_(src), 5)
    copy_gbs = 2.0 * src.numel() / (copy_ms * 1e-3) / 1e9
    del src, dst

    if args.secondary:
        progress("secondary kernels")
    extra = secondary(layers[0], args.bps, dev) if args.secondary else None

    progress("rate and quality of layer 0")
    rq = rate_and_quality(layers[0], args.bps)

    cpu = parity = None
    if args.cpu_baseline:
        import numpy as np
        xs0, encs0, ys0 = layers[0]
        # the last timed step's results for layer 0, and its inputs, on the host
        layer0_host = {
            "bits": np.concatenate([x.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, 256)
                                    for x in xs0]),
            "scale": np.concatenate([e["scale"].cpu().numpy() for e in encs0]),
            "idx": np.concatenate([e["idx"].cpu().numpy().reshape(-1, 256) for e in encs0]),
            "coset": np.concatenate([e["coset"].cpu().numpy().view(np.uint32).reshape(-1, 1)
                                     for e in encs0]),
            "rice_k": np.concatenate([e["rice_k"].cpu().numpy() for e in encs0]).astype(np.int64),
            "tile_bits": np.concatenate([e["tile_bits"].cpu().numpy().view(np.uint32)
                                         for e in encs0]).astype(np.int64),
            "y": np.concatenate([y.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, 256)
                                 for y in ys0]),
        }
        sx = workloads.small_fp32()
        sxd = torch.from_numpy(sx).to(dev)
        se = hq.hq_encode_tiles(sxd, "E8", 256, args.bps, 1)
        sy = hq.hq_decode_tiles(se["idx"], se["coset"], se["scale"], "E8", 256, 1, torch.bfloat16)
        torch.cuda.synchronize()
        small_host = {
            "x": sx, "scale": se["scale"].cpu().numpy(),
            "idx": se["idx"].cpu().numpy().reshape(-1, 256),
            "coset": se["coset"].cpu().numpy().view(np.uint32).reshape(-1, 1),
            "rice_k": se["rice_k"].cpu().numpy().astype(np.int64),
            "tile_bits": se["tile_bits"].cpu().numpy().view(np.uint32).astype(np.int64),
            "y": sy.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1, 256)}
        del sxd, se, sy
        progress("cpu baseline (oracle on the host)")
        cpu, par = cpu_baseline(layer0_host, small_host, args.bps)
        parity = {
            "rule": "indices and coset bits equal the oracle's on every block except oracle "
                    "near-ties (margin < 1e-6), scales equal except on bf16-midpoint tiles, "
                    "k and bits equal on matching tiles, bf16 decode of the GPU's indices "
                    "equal to the oracle's",
            "excused_mismatch_cap": "mismatches may only fall on oracle near-ties, at most 1e-5 "
                                    "of the blocks; near_ties counts the oracle's blocks with a "
                                    "margin below 1e-6, mismatches those that differ",
            "small_fp32_1024x1024": par["small"],
            "llama_layer0_all_seven": par["layer"]}

    # the dominant kernel's limiter: HBM when its traffic fraction is the
    # larger one, else VALU issue (when measured)
    bound = "hbm"
    if alu is not None and alu["frac"] > dominant["gbs"] / HBM_PEAK_GBS:
        bound = "alu"
    value = 2.0 * n_weights / (ms_per_step * 1e-3) / 1e9
    alg = (ENC_BYTES_PER_TILE + DEC_BYTES_PER_TILE) * n_tiles / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "E8 encode+decode throughput, bf16 GB/s in and % of HBM peak (1 GPU)",
        "value": round(value, 3),
        "unit": "GB/s (bf16 in)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {
            "workload": "llama3.1-8b-shaped 32-layer weight stack streamed through encode "
                        "then decode (E8, tile 256, auto scale)",
            "layers": args.layers, "weights": n_weights, "bps": args.bps, "tile": 256,
            "lattice": "E8", "input": "bf16", "output": "bf16",
            "schedule": ("pipelined: launch l encodes layer l and decodes layer l - 1 "
                         "(hq_encode_decode_batch, %d launches)" % (L + 1)) if pipe is not None
            else "sequential: per layer one encode launch, then one decode launch",
        },
        "pct_hbm_peak_algorithmic": round(100.0 * alg / HBM_PEAK_GBS, 3),
        "algorithmic_gbs": round(alg, 2),
        "roofline": dict({
            "kernel": dom_name,
            "bound": bound,
        }, **({"achieved": alu["achieved"], "peak": alu["peak"], "unit": alu["unit"],
               "frac": alu["frac"]} if bound == "alu" else
              {"achieved": round(dominant["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(dominant["gbs"] / HBM_PEAK_GBS, 4)}), **{
            "traffic": traffic,
            "traffic_unit": "measured HBM bytes per launch (null: kernel changed since the counters)",
            "algorithmic_bytes_per_launch": round(dominant["bytes_per_launch"]),
            "hbm": {"achieved": round(dominant["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(dominant["gbs"] / HBM_PEAK_GBS, 4)},
            "alu_issue": alu,
        }),
        "kernels": {k: {q: round(v, 3) for q, v in st.items()} for k, st in kern.items()},
        "host_wall_ms_per_step": round(head["host_wall_ms_per_step"], 3),
        "gpu_event_ms_per_step": round(head["gpu_event_ms_per_step"], 3),
        "sequential": {"ms_per_step": round(seq["ms_per_step"], 4),
                       "value": round(2.0 * n_weights / (seq["ms_per_step"] * 1e-3) / 1e9, 3),
                       "pct_hbm_peak_algorithmic": round(
                           100.0 * (ENC_BYTES_PER_TILE + DEC_BYTES_PER_TILE) * n_tiles /
                           (seq["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 3)},
        "pipelined_outputs_identical": same,
        "cache_cold": cold,
        "device_copy_gbs": round(copy_gbs, 1),
        "cpu_baseline": cpu,
        "parity": parity,
        "rate_and_quality": rq,
        "secondary": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
