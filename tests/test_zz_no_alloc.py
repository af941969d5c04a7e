"""hq_rate_noalloc (the entry point for callers that cannot allocate: its
scratch is a static device array of the library) against hq_rate with a
caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, packing and rate-only, with and without the encoder's rate
values given.  Everything must agree bit for bit."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
import hq_testlib as T

pytestmark = pytest.mark.gpu

from lattice_post_quantization_amd import hq  # noqa: E402  (fails loudly if unbuilt)


def _indices(rows, cols, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((rows, cols)) * 0.02
    w[:, ::53] *= 300.0
    x = T.bf16_device(workloads.f32_to_bf16_bits(w.astype(np.float32)), (rows, cols))
    return hq.hq_encode_tiles(x, "E8", 256, 4.0, seed)


def _same(a, b, pack):
    assert torch.equal(a["rice_k"], b["rice_k"])
    assert torch.equal(a["tile_bits"], b["tile_bits"])
    assert int(a["total_bits"][0]) == int(b["total_bits"][0])
    if pack:
        assert torch.equal(a["tile_word_offset"], b["tile_word_offset"])
        nw = int(a["tile_word_offset"][-1])
        assert torch.equal(a["stream"][:nw], b["stream"][:nw])


def test_rate_noalloc_matches_rate_with_workspace():
    # a large call first, then a smaller one: the second must not see the
    # first's sums in the shared scratch
    for rows, cols, seed in ((1024, 6144, 1), (37, 1280, 2)):
        enc = _indices(rows, cols, seed)
        torch.cuda.synchronize()
        print("case: hq_rate_noalloc %dx%d seed %d" % (rows, cols, seed), flush=True)
        for pack in (True, False):
            for given in (None, enc):
                ref = hq.hq_rate(enc["idx"], enc["coset"], "E8", 256, pack=pack,
                                 given=dict(given) if given is not None else None)
                got = hq.hq_rate(enc["idx"], enc["coset"], "E8", 256, pack=pack,
                                 given=dict(given) if given is not None else None, noalloc=True)
                torch.cuda.synchronize()
                _same(ref, got, pack)
                if pack and given is None:
                    T.host(got["stream"])      # readable on the host


def test_rate_noalloc_refusals():
    """Argument errors return before any device work, as for hq_rate."""
    lib = hq.lib()
    p = hq.make_params("E8", 256, 4.0)
    z = torch.zeros(256, dtype=torch.int8, device="cuda")
    k = torch.zeros(1, dtype=torch.uint8, device="cuda")
    b = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = torch.zeros(1, dtype=torch.int64, device="cuda")
    assert lib.hq_rate_noalloc(ctypes.byref(p), None, None, 0, None, None, None, None, 0, None,
                               None, None) == hq.HQ_OK
    assert lib.hq_rate_noalloc(ctypes.byref(p), z.data_ptr(), None, -1, k.data_ptr(),
                               b.data_ptr(), t.data_ptr(), None, 0, None, None,
                               None) == hq.HQ_EINVAL
    # packing needs the offsets
    s = torch.zeros(64, dtype=torch.int32, device="cuda")
    assert lib.hq_rate_noalloc(ctypes.byref(p), z.data_ptr(), None, 1, k.data_ptr(),
                               b.data_ptr(), t.data_ptr(), s.data_ptr(), 64, None, None,
                               None) == hq.HQ_EINVAL
