"""HyperQuant hot path on MI355X: HIP kernels behind a C ABI (include/hq.h)
and a thin Python binding (hq.py)."""

from .hq import (  # noqa: F401
    HQError, hq_decode_batch, hq_decode_tiles, hq_encode_batch, hq_encode_tiles, hq_kv_encode,
    hq_gemm, hq_gemm_batch, hq_gemv, hq_gemv_batch, hq_kv_scores, hq_rate, hq_unpack,
    hq_unpack_batch, lib, ckpt_save, ckpt_load, ckpt_entries,
)
