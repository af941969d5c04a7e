"""Checkpoint files of packed matrices (host code in the library): records
written and read back through the C ABI, with streams the oracle packs, and
the error codes of damaged, foreign and missing files."""

import ctypes
import os

import numpy as np
import pytest
import torch

from lattice_post_quantization_amd import hq
from oracle import codec, rice
import workloads


def _oracle_packed(rng, rows, cols, lattice="E8", tile=256, seed=3):
    w = rng.standard_normal((rows, cols)) * 0.02
    x = workloads.bf16_bits_to_f64(workloads.f32_to_bf16_bits(w.astype(np.float32)))
    ora = codec.encode(x, lattice, tile, 4.0, rht_seed=seed)
    cb = codec.coset_bits_per_tile(lattice, tile)
    idx = ora["idx"].reshape(-1, tile)
    _, _, words, off = rice.pack(idx, ora["coset"], cb)
    return ora, idx, words, off


def _save(path, name, words, off, scale, rows, cols, lattice="E8", tile=256, seed=3):
    packed = {"stream": torch.from_numpy(words.view(np.int32).copy()),
              "tile_word_offset": torch.from_numpy(off.astype(np.int64))}
    hq.ckpt_save(path, name, packed, torch.from_numpy(np.asarray(scale, np.float32)), rows, cols,
                 lattice=lattice, tile=tile, rht_seed=seed)


def test_round_trip_of_oracle_streams(tmp_path):
    """Three records (E8/256, D4/128, A2/64) come back bit for bit, and the
    oracle's own unpack of the loaded stream returns the encoded indices."""
    rng = np.random.default_rng(5)
    path = str(tmp_path / "layer.hqckpt")
    cases = [("q_proj", 37, 512, "E8", 256), ("k_proj", 16, 384, "D4", 128),
             ("v_proj", 3, 192, "A2", 64)]
    made = {}
    for name, rows, cols, lat, tile in cases:
        ora, idx, words, off = _oracle_packed(rng, rows, cols, lat, tile)
        _save(path, name, words, off, ora["scale"], rows, cols, lat, tile)
        made[name] = (ora, idx, words, off, lat, tile)
    ents = hq.ckpt_entries(path)
    assert [e["name"] for e in ents] == ["q_proj", "k_proj", "v_proj"]
    for name, rows, cols, lat, tile in cases:
        ora, idx, words, off, lat, tile = made[name]
        got = hq.ckpt_load(path, name)
        assert (got["rows"], got["cols"], got["lattice"], got["tile"]) == (rows, cols, lat, tile)
        assert got["n_tiles"] == idx.shape[0] and got["n_words"] == len(words)
        assert np.array_equal(got["stream"].numpy().view(np.uint32)[:len(words)], words)
        assert np.array_equal(got["tile_word_offset"].numpy(), off)
        assert np.array_equal(got["scale"].numpy(), ora["scale"].astype(np.float32))
        cb = codec.coset_bits_per_tile(lat, tile)
        back, cos, _ = rice.unpack(got["stream"].numpy().view(np.uint32), off, tile, cb)
        assert np.array_equal(back, idx)
        if cb:
            assert np.array_equal(cos, rice.coset_bit_rows(ora["coset"], cb))


def test_record_size_is_the_itemized_stored_rate(tmp_path):
    """A record's bytes are the oracle's itemized accounting of what it
    stores (fp32 scales, a uint64 tile word offset table, the packed stream
    with its word padding) plus the fixed 136-byte header and the zero bytes
    that align the scale and word arrays to 8 bytes."""
    rng = np.random.default_rng(8)
    path = str(tmp_path / "one.hqckpt")
    for name, rows, cols in (("even", 16, 512), ("odd", 7, 768)):
        ora, idx, words, off = _oracle_packed(rng, rows, cols)
        before = os.path.getsize(path) if os.path.exists(path) else 8   # file magic
        _save(path, name, words, off, ora["scale"], rows, cols)
        grown = os.path.getsize(path) - before
        it = codec.itemized_rate(ora["tile_bits"], "E8", 256, scale_bits=32, offset_bits=64)
        T, W = idx.shape[0], len(words)
        align = 8 * ((4 * T) % 8 + (4 * W) % 8)
        assert 8 * grown == it["total"] + 8 * 136 + align
        assert it["bps"] > codec.itemized_rate(ora["tile_bits"], "E8", 256)["bps"]


def test_error_codes(tmp_path):
    rng = np.random.default_rng(6)
    ora, idx, words, off = _oracle_packed(rng, 8, 512)
    path = str(tmp_path / "a.hqckpt")
    _save(path, "w", words, off, ora["scale"], 8, 512)
    # a taken name
    with pytest.raises(hq.HQError) as ex:
        _save(path, "w", words, off, ora["scale"], 8, 512)
    assert ex.value.code == hq.HQ_EINVAL
    # offsets that decrease, a shape that is not whole tiles
    bad = off.copy()
    bad[1], bad[2] = bad[2], bad[1]
    with pytest.raises(hq.HQError) as ex:
        _save(path, "x", words, bad, ora["scale"], 8, 512)
    assert ex.value.code == hq.HQ_EINVAL
    with pytest.raises(hq.HQError) as ex:
        _save(path, "x", words, off, ora["scale"], 8, 500)
    assert ex.value.code == hq.HQ_EINVAL
    # a shape whose product would leave int64 is refused, not wrapped
    e = hq.CkptEntry(b"big", hq.HQ_E8, 256, 4.0, 0, 1 << 40, 1 << 40, 16, 0)
    offs = np.zeros(17, np.int64)
    sc = np.zeros(16, np.float32)
    assert hq.lib().hq_ckpt_append(path.encode(), ctypes.byref(e), sc.ctypes.data,
                                   offs.ctypes.data, None) == hq.HQ_EINVAL
    # a missing record, a missing file, a directory that does not exist
    with pytest.raises(hq.HQError) as ex:
        hq.ckpt_load(path, "nope")
    assert ex.value.code == hq.HQ_ENOTFOUND
    with pytest.raises(hq.HQError) as ex:
        hq.ckpt_entries(str(tmp_path / "missing.hqckpt"))
    assert ex.value.code == hq.HQ_EIO
    with pytest.raises(hq.HQError) as ex:
        _save(str(tmp_path / "no" / "dir.hqckpt"), "w", words, off, ora["scale"], 8, 512)
    assert ex.value.code == hq.HQ_EIO
    # a file that is not a checkpoint: neither read nor appended to
    other = tmp_path / "other.bin"
    other.write_bytes(b"not a checkpoint file at all")
    for fn in (lambda: hq.ckpt_entries(str(other)),
               lambda: _save(str(other), "w", words, off, ora["scale"], 8, 512)):
        with pytest.raises(hq.HQError) as ex:
            fn()
        assert ex.value.code == hq.HQ_EFORMAT


def test_damage_is_detected(tmp_path):
    """One flipped payload bit fails the checksum; a cut file fails the
    record read (HQ_EFORMAT); the undamaged first record still loads."""
    rng = np.random.default_rng(7)
    path = str(tmp_path / "d.hqckpt")
    ora, idx, words, off = _oracle_packed(rng, 4, 512)
    _save(path, "first", words, off, ora["scale"], 4, 512)
    size_first = os.path.getsize(path)
    _save(path, "second", words, off, ora["scale"], 4, 512)
    raw = bytearray(open(path, "rb").read())
    flipped = bytearray(raw)
    flipped[size_first + 136 + 9] ^= 0x10      # inside the second record's payload
    p2 = str(tmp_path / "flip.hqckpt")
    open(p2, "wb").write(bytes(flipped))
    assert hq.ckpt_load(p2, "first")["n_words"] == len(words)
    with pytest.raises(hq.HQError) as ex:
        hq.ckpt_load(p2, "second")
    assert ex.value.code == hq.HQ_EFORMAT
    p3 = str(tmp_path / "cut.hqckpt")
    open(p3, "wb").write(bytes(raw[:-5]))
    with pytest.raises(hq.HQError) as ex:
        hq.ckpt_load(p3, "second")
    assert ex.value.code == hq.HQ_EFORMAT


def test_empty_matrix_record(tmp_path):
    path = str(tmp_path / "e.hqckpt")
    packed = {"stream": torch.zeros(1, dtype=torch.int32),
              "tile_word_offset": torch.zeros(1, dtype=torch.int64)}
    hq.ckpt_save(path, "empty", packed, torch.zeros(0), 0, 256)
    got = hq.ckpt_load(path, "empty")
    assert got["n_tiles"] == 0 and got["n_words"] == 0 and got["rows"] == 0


@pytest.mark.gpu
def test_device_pack_file_unpack_round_trip(tmp_path):
    """Encode on the GPU, pack, write the record, read it back, copy to the
    device and unpack: indices and cosets are the encoder's, and decoding
    with the loaded scales gives the same bits as with the originals."""
    rng = np.random.default_rng(8)
    rows, cols = 300, 4096
    bits = workloads.f32_to_bf16_bits((rng.standard_normal((rows, cols)) * 0.02).astype(np.float32))
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).reshape(rows, cols).cuda()
    print("case: ckpt round trip E8/256 %dx%d" % (rows, cols), flush=True)
    e = hq.hq_encode_tiles(x, "E8", 256, 4.0, 11)
    r = hq.hq_rate(e["idx"], e["coset"], "E8", 256, pack=True)
    path = str(tmp_path / "dev.hqckpt")
    hq.ckpt_save(path, "w", r, e["scale"], rows, cols, rht_seed=11)
    got = hq.ckpt_load(path, "w", device=x.device)
    u = hq.hq_unpack(got["stream"], got["tile_word_offset"], "E8", 256)
    torch.cuda.synchronize()
    assert torch.equal(u["idx"].reshape(-1), e["idx"].reshape(-1))
    assert torch.equal(u["coset"].reshape(-1), e["coset"].reshape(-1))
    y0 = hq.hq_decode_tiles(e["idx"], e["coset"], e["scale"], "E8", 256, 11, torch.bfloat16)
    y1 = hq.hq_decode_tiles(u["idx"].reshape(e["idx"].shape), u["coset"].reshape(e["coset"].shape),
                            got["scale"].reshape(e["scale"].shape), "E8", 256, got["rht_seed"],
                            torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.gpu
def test_layer_checkpoint_round_trip(tmp_path):
    """A Llama-3.1-8B-shaped layer as the benchmark draws it: seven matrices
    encoded and packed in one batched call each, written as seven records of
    one file, read back onto the device and decoded by one batched
    hq_unpack: every index and coset equals the encoder's."""
    dev = torch.device("cuda")
    xs = [workloads.llama_stack_torch(0, m, dev) for m in range(len(workloads.LLAMA_LAYER))]
    print("case: layer checkpoint (seven matrices)", flush=True)
    encs = hq.hq_encode_batch(xs, "E8", 256, 4.0, 0)
    packs = hq.hq_rate_batch(encs, "E8", 256, pack=True, given=True)
    path = str(tmp_path / "layer0.hqckpt")
    names = [name for name, _, _ in workloads.LLAMA_LAYER]
    for name, x, e, pk in zip(names, xs, encs, packs):
        hq.ckpt_save(path, name, pk, e["scale"], x.shape[0], x.shape[1])
    assert [e["name"] for e in hq.ckpt_entries(path)] == names
    loaded = [hq.ckpt_load(path, name, device=dev) for name in names]
    outs = hq.hq_unpack_batch(loaded, "E8", 256)
    torch.cuda.synchronize()
    for name, e, got, u in zip(names, encs, loaded, outs):
        assert torch.equal(u["idx"].reshape(-1), e["idx"].reshape(-1)), name
        assert torch.equal(u["coset"].reshape(-1), e["coset"].reshape(-1)), name
        assert torch.equal(got["scale"].reshape(-1), e["scale"].reshape(-1)), name
