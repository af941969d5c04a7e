"""HyperQuant hot path on MI355X: HIP kernels behind a C ABI (include/hq.h)
and a thin Python binding (hq.py)."""

from .hq import (  # noqa: F401
    HQError, ckpt_entries, ckpt_load, ckpt_save, hq_decode_batch, hq_decode_tiles,
    hq_encode_batch, hq_encode_tiles, hq_gemm, hq_gemm_batch, hq_gemv, hq_gemv_batch,
    hq_kv_attention, hq_kv_encode, hq_kv_scores, hq_rate, hq_rate_batch, hq_unpack,
    hq_unpack_batch, lib,
)
