"""Rice coding of stripped lattice indices (oracle side; test infrastructure).

[arXiv abstract] item (iii) and [ICLR abstract]: after the lossless strip the
remaining index integers are carried by a variable-length Rice code (within
about 0.1 bps of the lattice's rate-distortion ideal), under one itemized rate
accounting; [issue] "Additional context" names a packed, Rice-coded
lattice-index checkpoint format.  The pages fix none of the code's details.

Readings:
* signed integers map to codes by the zigzag map zeta(z) = 2z (z >= 0),
  -2z - 1 (z < 0);
* one Rice parameter k per tile, k in [0, 15], chosen to minimise the tile's
  payload, smallest k on ties; a code is floor(zeta / 2^k) one-bits, a zero
  bit, then the k low bits of zeta, least significant first;
* a tile costs 4 bits for k, its coset bits (E8: one per 8-block, A2: one per
  pair, D4/Z: none) and the Rice payload;
* packed layout: per tile, k (4 bits), coset bits (block j at position j),
  codes in index order; bit j of the stream is bit (j mod 32) of 32-bit word
  j div 32; every tile starts on a word boundary, zero-padded; the tile word
  offsets are the exclusive prefix sum of ceil(tile_bits / 32).
"""

import numpy as np

K_MAX = 15
K_FIELD_BITS = 4


def zigzag(z):
    z = np.asarray(z, np.int64)
    return np.where(z >= 0, 2 * z, -2 * z - 1)


def unzigzag(q):
    q = np.asarray(q, np.int64)
    return np.where(q % 2 == 0, q // 2, -(q + 1) // 2)


def code_length(zeta, k):
    """Length in bits of the Rice code of zeta with parameter k."""
    return (np.asarray(zeta, np.int64) >> k) + 1 + k


def payload_bits(idx):
    """L[t, k] = sum over the tile's indices of code_length(zeta, k), k=0..15."""
    zeta = zigzag(idx)
    return np.stack([code_length(zeta, k).sum(axis=-1) for k in range(K_MAX + 1)],
                    axis=-1)


def best_k(idx):
    """Per-tile (k, payload) with k = argmin_k L(k), lowest k on ties."""
    L = payload_bits(idx)
    k = np.argmin(L, axis=-1)
    return k, np.take_along_axis(L, k[..., None], axis=-1)[..., 0]


def tile_bits(idx, coset_bits_per_tile):
    """(k, total bits) per tile: 4 + coset bits + minimal Rice payload."""
    k, pay = best_k(idx)
    return k, K_FIELD_BITS + coset_bits_per_tile + pay


# ------------------------------------------------------------------ packing

def _tile_bitstring(idx_row, coset_row_bits, k):
    zeta = zigzag(idx_row)
    q = zeta >> k
    lens = q + 1 + k
    head = [(k >> b) & 1 for b in range(K_FIELD_BITS)] + list(coset_row_bits)
    total = len(head) + int(lens.sum())
    bits = np.zeros(total, np.uint8)
    bits[:len(head)] = head
    start = len(head) + np.concatenate([[0], np.cumsum(lens)[:-1]])
    # unary part: q ones at start .. start+q-1
    ones = np.repeat(start, q) + (np.arange(q.sum()) - np.repeat(np.cumsum(q) - q, q))
    bits[ones] = 1
    # remainder: k low bits after the terminating zero, LSB first
    for b in range(k):
        bits[start + q + 1 + b] = (zeta >> b) & 1
    return bits


def coset_bit_rows(coset_words, n_bits):
    """Unpack per-tile coset words (uint32, LSB-first) into 0/1 rows."""
    cw = np.asarray(coset_words, np.uint64).reshape(len(coset_words), -1)
    j = np.arange(n_bits)
    return ((cw[:, j // 32] >> (j % 32).astype(np.uint64)) & np.uint64(1)).astype(np.uint8)


def pack(idx, coset_words, coset_bits_per_tile):
    """Pack tiles into the word stream.

    Returns (k, tile_bits, words uint32, tile_word_offset int64[n_tiles+1]).
    """
    idx = np.asarray(idx, np.int64)
    n_tiles = idx.shape[0]
    k, tb = tile_bits(idx, coset_bits_per_tile)
    cbits = (coset_bit_rows(coset_words, coset_bits_per_tile)
             if coset_bits_per_tile else np.zeros((n_tiles, 0), np.uint8))
    nwords = (tb + 31) // 32
    off = np.concatenate([[0], np.cumsum(nwords)]).astype(np.int64)
    words = np.zeros(int(off[-1]), np.uint32)
    for t in range(n_tiles):
        bits = _tile_bitstring(idx[t], cbits[t], int(k[t]))
        assert bits.size == tb[t]
        padded = np.zeros(int(nwords[t]) * 32, np.uint8)
        padded[:bits.size] = bits
        by = np.packbits(padded, bitorder="little")
        words[off[t]:off[t + 1]] = by.view("<u4")
    return k, tb, words, off


def unpack(words, tile_word_offset, n_idx, coset_bits_per_tile):
    """Inverse of pack: (idx int64 (T, n_idx), coset_bits (T, c), k (T,))."""
    words = np.asarray(words, np.uint32)
    off = np.asarray(tile_word_offset, np.int64)
    n_tiles = len(off) - 1
    idx = np.zeros((n_tiles, n_idx), np.int64)
    cos = np.zeros((n_tiles, coset_bits_per_tile), np.uint8)
    ks = np.zeros(n_tiles, np.int64)
    for t in range(n_tiles):
        seg = words[off[t]:off[t + 1]].astype("<u4").view(np.uint8)
        bits = np.unpackbits(seg, bitorder="little")
        pos = 0
        k = int(sum(int(bits[pos + b]) << b for b in range(K_FIELD_BITS)))
        pos += K_FIELD_BITS
        cos[t] = bits[pos:pos + coset_bits_per_tile]
        pos += coset_bits_per_tile
        for i in range(n_idx):
            q = 0
            while bits[pos] == 1:
                q += 1
                pos += 1
            pos += 1
            r = 0
            for b in range(k):
                r |= int(bits[pos + b]) << b
            pos += k
            idx[t, i] = (q << k) | r
        ks[t] = k
    return unzigzag(idx), cos, ks
