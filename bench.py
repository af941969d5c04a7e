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

# Measured HBM bytes per tile (rocprofv3 FETCH_SIZE and WRITE_SIZE per
# dispatch, each scaled by what the same counter reads for a copy of known
# size) and VALU lane-operations per weight (SQ_INSTS_VALU per dispatch x 64
# lanes); the runs are summarised in profiles/.  They describe the kernels
# built from the sources with this sha256 and are reported only while the
# sources still match.
KERNEL_SOURCES = ("hq_e8fast.hip", "hq_lanes.h", "hq_device.h", "hq_internal.h")
MEASURED_TRAFFIC = {
    "sources_sha256": "aecf7cb8364cdf9ce554d40ee42718e6255ee38f73e15f73f785749b1b9b001a",
    "encode": {"read": 513.87, "write": 269.32},
    "decode": {"read": 264.28, "write": 512.00},
    "valu_lane_ops_per_weight": {"encode": 36.51, "decode": 11.92},
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
                    help="time the oracle on a sample of the workload (rank 0, N=1)")
    ap.add_argument("--cpu-sample-stride", type=int, default=4,
                    help="oracle sample: every k-th tile of layer 0")
    ap.add_argument("--secondary", type=int, default=1,
                    help="after the timed steps, also time the pack pass and the KV path "
                         "(reported beside the headline, never in it)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a kernel of "
                         "known traffic that scales the profiler's byte counters)")
    return ap.parse_args()


# ------------------------------------------------------------ CPU baseline

def _oracle_chunk(args):
    tiles, seed, bps = args
    from threadpoolctl import threadpool_limits
    from oracle import codec
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        e = codec.encode(tiles, "E8", 256, bps, rht_seed=seed)
        codec.decode(e["idx"], e["coset"], e["scale"], "E8", 256, seed)
        return time.perf_counter() - t0


def cpu_baseline(stride, bps):
    """The oracle (fp64 NumPy, unmodified) on every stride-th tile of a
    host-drawn layer of the same shapes and distribution, spread over the
    host's cores (one single-threaded process each)."""
    import multiprocessing as mp

    import numpy as np

    import workloads
    chunks = []
    n_w = 0
    for m in range(7):
        bits = workloads.llama_matrix(m, layer=0)
        t = workloads.bf16_bits_to_f64(bits.reshape(-1, 256)[::stride])
        n_w += t.size
        chunks.extend(np.array_split(t, max(1, len(t) // 2048)))
    procs = min(os.cpu_count() or 1, 16)
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        t0 = time.perf_counter()
        pool.map(_oracle_chunk, [(c, 0, bps) for c in chunks], chunksize=1)
        wall = time.perf_counter() - t0
    return {
        "value": round(2.0 * n_w / wall / 1e9, 6),
        "unit": "GB/s (bf16 in)",
        "cores": procs,
        "kind": "oracle",
        "sample": "every %dth 256-weight tile of one host-drawn layer of the same "
                  "shapes and distribution (%d weights), E8 4 bps encode + decode, "
                  "%d single-threaded processes, %.1f s wall" % (stride, n_w, procs, wall),
    }


# ------------------------------------------------------------------- GPU

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

    # the stream decoder on the same streams
    unp = [hq.hq_unpack(o["stream"], o["tile_word_offset"], "E8", 256) for o in outs]

    def unpack_layer():
        for o, u in zip(outs, unp):
            hq.hq_unpack(o["stream"], o["tile_word_offset"], "E8", 256, out=u)

    ms_u = time_calls(unpack_layer, 10)
    torch.cuda.synchronize()
    same = all(torch.equal(u["idx"].view(-1), e["idx"].view(-1)) for u, e in zip(unp, encs))
    # the seven streams in one call (one lane per tile: together they fill the GPU)
    unp_b = hq.hq_unpack_batch(outs, "E8", 256)

    def unpack_layer_batched():
        hq.hq_unpack_batch(outs, "E8", 256, outs=unp_b)

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
    for m in (32, 128):
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

    # variants on the same layer's weights: per-tile rate control (the
    # generic kernel searches about a dozen scales per tile) and tile 512
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
        "workload": "the same layer's seven matrices (bf16) through the generic kernels",
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

    cpu = cpu_baseline(args.cpu_sample_stride, args.bps) if args.cpu_baseline else None

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

    # events for the timed region are created up front (creation is a host
    # call that would otherwise sit between kernel launches)
    n_ev = 2 * len(layers) * args.steps
    ev = {"enc": [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)],
          "dec": [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)],
          "enc_tiles": [], "dec_tiles": []}
    cursor = {"enc": 0, "dec": 0}

    def mark(kind):
        ev[kind][cursor[kind]].record()
        cursor[kind] += 1

    def step(timed):
        # one launch encodes a layer's seven projections, one launch decodes them
        for layer, (xs, encs, ys) in enumerate(layers):
            if timed:
                mark("enc")
            hq.hq_encode_batch(xs, "E8", 256, args.bps, layer, outs=encs)
            if timed:
                mark("enc")
                ev["enc_tiles"].append(tiles_per_layer[layer])
                mark("dec")
            hq.hq_decode_batch(encs, "E8", 256, layer, torch.bfloat16, outs=ys)
            if timed:
                mark("dec")
                ev["dec_tiles"].append(tiles_per_layer[layer])

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # timed region: whole steps, bracketed by synchronisation
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        step(True)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps

    def kernel_stats(name, tiles_key, bytes_per_tile):
        evs = ev[name][:cursor[name]]
        durs = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(len(evs) // 2)]
        tiles = ev[tiles_key]
        tot_ms = sum(durs)
        tot_bytes = sum(t * bytes_per_tile for t in tiles)
        return {"launches": len(durs), "avg_us": 1e3 * tot_ms / len(durs),
                "sum_ms_per_step": tot_ms / args.steps,
                "gbs": tot_bytes / (tot_ms * 1e-3) / 1e9}

    enc = kernel_stats("enc", "enc_tiles", ENC_BYTES_PER_TILE)
    dec = kernel_stats("dec", "dec_tiles", DEC_BYTES_PER_TILE)
    dominant = enc if enc["sum_ms_per_step"] >= dec["sum_ms_per_step"] else dec
    dom_name = "encode" if dominant is enc else "decode"

    tiles_per_launch = sum(ev["enc_tiles"]) / len(ev["enc_tiles"])
    traffic = alu = None
    if kernel_sources_sha256() == MEASURED_TRAFFIC["sources_sha256"]:
        t = MEASURED_TRAFFIC[dom_name]
        traffic = round((t["read"] + t["write"]) * tiles_per_launch)
        # the same launches against the VALU issue roof
        ops = MEASURED_TRAFFIC["valu_lane_ops_per_weight"][dom_name] * 256 * tiles_per_launch
        achieved = ops / (dominant["avg_us"] * 1e-6)
        alu = {"achieved": round(achieved / 1e12, 2), "peak": round(VALU_PEAK_LANE_OPS / 1e12, 2),
               "unit": "T VALU lane-ops/s (issued)", "frac": round(achieved / VALU_PEAK_LANE_OPS, 4),
               "lane_ops_per_weight": MEASURED_TRAFFIC["valu_lane_ops_per_weight"][dom_name]}

    extra = secondary(layers[0], args.bps, dev) if args.secondary else None

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
        },
        "pct_hbm_peak_algorithmic": round(100.0 * alg / HBM_PEAK_GBS, 3),
        "algorithmic_gbs": round(alg, 2),
        "roofline": {
            "kernel": dom_name,
            "bound": "hbm",
            "achieved": round(dominant["gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dominant["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (null: kernel changed since the counters)",
            "algorithmic_bytes_per_launch": round(
                (ENC_BYTES_PER_TILE if dom_name == "encode" else DEC_BYTES_PER_TILE) * tiles_per_launch),
            "alu_issue": alu,
        },
        "kernels": {
            "encode": {k: round(v, 3) for k, v in enc.items()},
            "decode": {k: round(v, 3) for k, v in dec.items()},
        },
        "host_wall_ms_per_step": round(wall * 1e3 / args.steps, 3),
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 3),
        "cpu_baseline": cpu,
        "secondary": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
