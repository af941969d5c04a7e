"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it only draws numbers and
casts them to the storage types.  The pages measure on Llama-3.1-8B weights,
WikiText-103, C4 and LTX-2, none of which is available; these generators stand
in for them with the shapes of a Llama-3.1-8B decoder layer (hidden 4096,
8 KV heads x 128, intermediate 14336, 32 layers) and Gaussian entries with
planted outliers.

Workloads (n = tile size):
  small_fp32   1024x1024 fp32, N(0,1), numpy default_rng(0); n=256, E8.
  llama_layer  the seven projections of one decoder layer in bf16,
               N(0, 0.02^2), with round(0.001 * in) input columns replaced by
               10 * Student-t(4) outliers; matrix m of layer l is drawn from
               default_rng(SeedSequence(l).spawn(7)[m]).
  llama_stack  32 such layers, drawn on the GPU with a torch generator seeded
               by the layer index (so 14 GB need not cross PCIe).
  sweep_matrix one 4096x14336 bf16 N(0, 0.02^2) matrix, default_rng(0).
  kv_layer     K and V, bf16 [8, 32768, 128], N(0,1), plus per-(head, channel)
               offsets N(0, 2^2) on 4 of the 128 channels, queries N(0,1).
"""

import numpy as np

LLAMA_LAYER = (
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336),
)
LLAMA_LAYERS = 32


def f32_to_bf16_bits(a):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b):
    u = np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def small_fp32(seed=0, shape=(1024, 1024)):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def llama_matrix(m, layer=0, shape=None):
    """bf16 bits (uint16) of projection m (0..6) of decoder layer `layer`.

    `shape` overrides (rows, cols) for reduced test sizes (same recipe)."""
    name, rows, cols = LLAMA_LAYER[m]
    if shape is not None:
        rows, cols = shape
    rng = np.random.default_rng(np.random.SeedSequence(layer).spawn(7)[m])
    w = rng.standard_normal((rows, cols)) * 0.02
    n_out = int(round(0.001 * cols))
    if n_out:
        col = rng.choice(cols, size=n_out, replace=False)
        w[:, col] = 10.0 * rng.standard_t(4, size=(rows, n_out))
    return f32_to_bf16_bits(w.astype(np.float32))


def sweep_matrix(seed=0, shape=(4096, 14336)):
    w = np.random.default_rng(seed).standard_normal(shape) * 0.02
    return f32_to_bf16_bits(w.astype(np.float32))


def kv_layer(seed=0, heads=8, seq=32768, dim=128, n_offset_channels=4):
    """(K bits, V bits) as uint16 [heads, seq, dim]."""
    ss = np.random.SeedSequence(seed).spawn(3)
    out = []
    ch_rng = np.random.default_rng(ss[2])
    channels = ch_rng.choice(dim, size=n_offset_channels, replace=False)
    for t in range(2):
        rng = np.random.default_rng(ss[t])
        a = rng.standard_normal((heads, seq, dim))
        off = rng.normal(0.0, 2.0, size=(heads, n_offset_channels))
        a[:, :, channels] += off[:, None, :]
        out.append(f32_to_bf16_bits(a.astype(np.float32)))
    return out[0], out[1]


def kv_queries(seed=3, count=4096, dim=128):
    return np.random.default_rng(seed).standard_normal((count, dim))


def llama_stack_torch(layer, m, device, dtype=None):
    """Matrix m of layer `layer` for the 32-layer stack, drawn on `device`.

    Same distribution as llama_matrix (different stream: torch's generator
    seeded with 1000 * layer + m)."""
    import torch
    name, rows, cols = LLAMA_LAYER[m]
    g = torch.Generator(device=device)
    g.manual_seed(1000 * layer + m)
    w = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * 0.02
    n_out = int(round(0.001 * cols))
    col = torch.randperm(cols, generator=g, device=device)[:n_out]
    # Student-t(4) = N / sqrt(chi2_4 / 4), chi2_4 = sum of 4 squared normals
    nrm = torch.randn((rows, n_out), generator=g, device=device)
    chi = (torch.randn((rows, n_out, 4), generator=g, device=device) ** 2).sum(-1)
    w[:, col] = 10.0 * nrm / torch.sqrt(chi / 4.0)
    return w.to(torch.bfloat16 if dtype is None else dtype)
