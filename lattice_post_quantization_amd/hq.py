"""Python binding of libhq.so (the HyperQuant hot path on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/hq.h.  PyTorch provides device memory and
the current HIP stream.  The names mirror the C entry points.

The library must be built first (`python -m lattice_post_quantization_amd.build`);
a missing library raises instead of falling back to anything else.
"""

import ctypes
import math
import os

import torch  # loads the HIP runtime first, so libhq.so binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhq.so")

HQ_OK, HQ_EINVAL, HQ_ERANGE, HQ_EDEVICE, HQ_EUNSUPPORTED = 0, -1, -2, -3, -4
HQ_EIO, HQ_EFORMAT, HQ_ENOTFOUND = -5, -6, -7
HQ_Z, HQ_A2, HQ_D4, HQ_E8 = 1, 2, 4, 8
HQ_F32, HQ_BF16 = 0, 1
HQ_SCALE_AUTO, HQ_DITHER, HQ_WANT_COORDS, HQ_RATE_CONTROL, HQ_RATE_GIVEN = 1, 2, 4, 8, 16
HQ_IDX16 = 32
HQ_ST_NONFINITE, HQ_ST_OVERFLOW, HQ_ST_STREAM_FULL, HQ_ST_CORRUPT = 1, 2, 4, 8

LATTICES = {"E8": HQ_E8, "D4": HQ_D4, "A2": HQ_A2, "Z": HQ_Z}


class HQError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__("%s: %s (%d)" % (what, status_string(code), code))


class Params(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("lattice", ctypes.c_int32),
        ("tile", ctypes.c_int32),
        ("bps", ctypes.c_float),
        ("rht_seed", ctypes.c_uint32),
        ("dither_seed", ctypes.c_uint32),
        ("dither_base", ctypes.c_int64),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


def make_params(lattice="E8", tile=256, bps=4.0, rht_seed=0, flags=0,
                dither_seed=0, dither_base=0):
    lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
    return Params(ctypes.sizeof(Params), lat, int(tile), float(bps), int(rht_seed),
                  int(dither_seed), int(dither_base), int(flags), 0)


class EncodeItem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("scale", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("coset", ctypes.c_void_p),
                ("rice_k", ctypes.c_void_p), ("tile_bits", ctypes.c_void_p)]


class GemvItem(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("coset", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p)]


class CkptEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("lattice", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("bps", ctypes.c_float), ("rht_seed", ctypes.c_uint32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("n_tiles", ctypes.c_int64),
                ("n_words", ctypes.c_uint64)]


class DecodeItem(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("coset", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("y", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _U32, _U64, _SZ = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                               ctypes.c_uint64, ctypes.c_size_t)
_PP = ctypes.POINTER(Params)

_SIGNATURES = {
    "hq_ckpt_append": (_I32, [ctypes.c_char_p, _P, _P, _P, _P]),
    "hq_ckpt_count": (_I32, [ctypes.c_char_p, _P]),
    "hq_ckpt_entry_at": (_I32, [ctypes.c_char_p, _I32, _P]),
    "hq_ckpt_read": (_I32, [ctypes.c_char_p, ctypes.c_char_p, _P, _P, _P, _P, _I64, _U64]),
    "hq_encode_tiles": (_I32, [_PP, _P, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "hq_decode_tiles": (_I32, [_PP, _P, _P, _P, _I64, _I64, _P, _I32, _P, _P]),
    "hq_rate": (_I32, [_PP, _P, _P, _I64, _P, _P, _P, _P, _U64, _P, _P, _SZ, _P, _P]),
    "hq_unpack": (_I32, [_PP, _P, _P, _I64, _P, _P, _P, _P, _P]),
    "hq_unpack_batch": (_I32, [_PP, _I32, _P, _P, _P]),
    "hq_gemv": (_I32, [_PP, _P, _P, _P, _I64, _I64, _P, _I32, _P, _P, _SZ, _P, _P]),
    "hq_gemv_workspace_bytes": (_SZ, [_I64, _I64, _I32]),
    "hq_gemm": (_I32, [_PP, _P, _P, _P, _I64, _I64, _P, _I32, _P, _P, _SZ, _P, _P]),
    "hq_gemm_workspace_bytes": (_SZ, [_I64, _I64, _I32]),
    "hq_gemm_batch": (_I32, [_PP, _I32, _P, _I32, _P, _SZ, _P, _P]),
    "hq_gemm_batch_workspace_bytes": (_SZ, [_I32, _P, _I32]),
    "hq_gemv_batch": (_I32, [_PP, _I32, _P, _I32, _P, _SZ, _P, _P]),
    "hq_rate_batch": (_I32, [_PP, _I32, _P, _P, _SZ, _P, _P]),
    "hq_rate_batch_workspace_bytes": (_SZ, [_I32, _P]),
    "hq_gemv_batch_workspace_bytes": (_SZ, [_I32, _P, _I32]),
    "hq_kv_scores": (_I32, [_PP, _P, _I64, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "hq_kv_scores_workspace_bytes": (_SZ, [_I64]),
    "hq_kv_attention": (_I32, [_PP, _P, _P, _P, _PP, _P, _P, _P, _I64, _I64, _P, _I64,
                               ctypes.c_float, _P, _P, _SZ, _P]),
    "hq_kv_attention_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "hq_kv_encode": (_I32, [_PP, _P, _I32, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "hq_encode_batch": (_I32, [_PP, _I32, _I32, _P, _P, _P]),
    "hq_decode_batch": (_I32, [_PP, _I32, _I32, _P, _P, _P]),
    "hq_encode_decode_batch": (_I32, [_PP, _I32, _I32, _P, _PP, _I32, _I32, _P, _P, _P]),
    "hq_rate_noalloc": (_I32, [_PP, _P, _P, _I64, _P, _P, _P, _P, _U64, _P, _P, _P]),
    "hq_coset_words": (_I32, [_PP]),
    "hq_rate_workspace_bytes": (_SZ, [_I64]),
    "hq_status_string": (ctypes.c_char_p, [_I32]),
    "hq_splitmix64": (_U64, [_U64]),
    "hq_rht_signs": (_I32, [_U32, _I32, _P]),
    "hq_scale_constant": (_I32, [_PP, ctypes.POINTER(ctypes.c_double)]),
    "hq_version": (_I32, []),
}


def lib():
    """The loaded libhq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhq.so is not built (%s); run "
                               "python -m lattice_post_quantization_amd.build" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def status_string(code):
    return lib().hq_status_string(int(code)).decode()


def _check(code, what):
    if code != HQ_OK:
        raise HQError(code, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return HQ_BF16
    if dt == torch.float32:
        return HQ_F32
    raise ValueError("dtype must be bfloat16 or float32")


def _device_tensor(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def coset_words(lattice="E8", tile=256):
    p = make_params(lattice, tile)
    return int(lib().hq_coset_words(ctypes.byref(p)))


def rate_workspace_bytes(n_tiles):
    return int(lib().hq_rate_workspace_bytes(int(n_tiles)))


def rht_signs(seed, n):
    import numpy as np
    out = np.zeros(n, np.int8)
    _check(lib().hq_rht_signs(int(seed), int(n), out.ctypes.data_as(ctypes.c_void_p)),
           "hq_rht_signs")
    return out


def scale_constant(lattice, bps):
    p = make_params(lattice, 256 if lattice == "E8" else 128, bps)
    out = ctypes.c_double()
    _check(lib().hq_scale_constant(ctypes.byref(p), ctypes.byref(out)), "hq_scale_constant")
    return out.value


def splitmix64(key):
    return int(lib().hq_splitmix64(int(key)))


def _idx_flag(idx):
    """HQ_IDX16 for int16 index tensors (the int16 index mode), else 0."""
    if idx.dtype == torch.int16:
        return HQ_IDX16
    if idx.dtype != torch.int8:
        raise TypeError("indices must be int8 (or int16 in the int16 index mode)")
    return 0


def hq_encode_tiles(x, lattice="E8", tile=256, bps=4.0, rht_seed=0, scale=None,
                    want_coords=False, status=None, out=None, rate_control=False,
                    idx16=False):
    """Encode a row-major (rows, cols) bf16/fp32 device matrix.

    scale=None selects auto scales (returned); otherwise a float32 device
    tensor of per-tile scales.  Returns a dict of device tensors: scale,
    idx (int8, like x; int16 with idx16), coset (int32 words, (n_tiles, w)),
    rice_k (uint8), tile_bits (int32 holding uint32), coords (int16, if
    requested).  `out` may supply preallocated tensors under the same keys.
    rate_control: per-tile scales so that each tile fits floor(bps * tile)
    bits (auto scales only; the chosen scales are returned).
    idx16: the int16 index mode (HQ_IDX16), for rates whose indices leave
    int8."""
    _device_tensor(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D (rows, cols)")
    rows, cols = x.shape
    dev = x.device
    n_tiles = rows * cols // tile if cols % tile == 0 else 0
    w = coset_words(lattice, tile)
    o = dict(out or {})
    flags = ((HQ_SCALE_AUTO if scale is None else 0) | (HQ_WANT_COORDS if want_coords else 0) |
             (HQ_RATE_CONTROL if rate_control else 0) | (HQ_IDX16 if idx16 else 0))
    if scale is None:
        scale = o.get("scale")
        if scale is None:
            scale = torch.empty(n_tiles, dtype=torch.float32, device=dev)
    else:
        _device_tensor(scale, "scale")
    idx = o.get("idx")
    if idx is None:
        idx = torch.empty((rows, cols), dtype=torch.int16 if idx16 else torch.int8, device=dev)
    elif (idx.dtype == torch.int16) != bool(idx16):
        raise TypeError("out['idx'] must be int16 exactly when idx16 is set")
    coset = o.get("coset")
    if coset is None:
        coset = torch.empty((n_tiles, max(w, 1)), dtype=torch.int32, device=dev)
    rice_k = o.get("rice_k")
    if rice_k is None:
        rice_k = torch.empty(n_tiles, dtype=torch.uint8, device=dev)
    tile_bits = o.get("tile_bits")
    if tile_bits is None:
        tile_bits = torch.empty(n_tiles, dtype=torch.int32, device=dev)
    coords = None
    if want_coords:
        coords = o.get("coords")
        if coords is None:
            coords = torch.empty((rows, cols), dtype=torch.int16, device=dev)
    p = make_params(lattice, tile, bps, rht_seed, flags)
    code = lib().hq_encode_tiles(ctypes.byref(p), _ptr(x), _dtype_code(x.dtype), rows, cols,
                                 _ptr(scale), _ptr(idx), _ptr(coset), _ptr(rice_k),
                                 _ptr(tile_bits), _ptr(coords), _ptr(status), _stream(dev))
    _check(code, "hq_encode_tiles")
    res = {"scale": scale, "idx": idx, "coset": coset, "rice_k": rice_k, "tile_bits": tile_bits}
    if want_coords:
        res["coords"] = coords
    return res


def hq_decode_tiles(idx, coset, scale, lattice="E8", tile=256, rht_seed=0,
                    out_dtype=torch.bfloat16, dither_seed=None, dither_base=0,
                    status=None, out=None):
    """Decode stripped indices back to weights (rows, cols) of out_dtype
    (int16 indices select the int16 index mode)."""
    _device_tensor(idx, "idx")
    _device_tensor(scale, "scale")
    if coset is not None:
        _device_tensor(coset, "coset")
    rows, cols = idx.shape
    y = out if out is not None else torch.empty((rows, cols), dtype=out_dtype, device=idx.device)
    flags = (HQ_DITHER if dither_seed is not None else 0) | _idx_flag(idx)
    p = make_params(lattice, tile, 4.0, rht_seed, flags,
                    0 if dither_seed is None else dither_seed, dither_base)
    code = lib().hq_decode_tiles(ctypes.byref(p), _ptr(idx), _ptr(coset), _ptr(scale), rows, cols,
                                 _ptr(y), _dtype_code(y.dtype), _ptr(status), _stream(idx.device))
    _check(code, "hq_decode_tiles")
    return y


def hq_rate(idx, coset, lattice="E8", tile=256, pack=False, capacity_words=None,
            status=None, out=None, given=None, noalloc=False):
    """Rice parameters and bit lengths per tile; optionally the packed stream.

    noalloc: call hq_rate_noalloc (the library's static scratch instead of a
    workspace; the outputs are still allocated here unless given in `out`).

    given: the encoder's result for these indices (a dict with rice_k and
    tile_bits, as hq_encode_tiles returns): HQ_RATE_GIVEN, the rate pass
    then reads tile_bits instead of recomputing both from the indices.
    Returns dict: rice_k, tile_bits, total_bits (int64 device scalar) and, when
    packing, stream (int32 words), tile_word_offset (int64, n_tiles + 1).
    int16 indices select the int16 index mode."""
    _device_tensor(idx, "idx")
    dev = idx.device
    n_tiles = idx.numel() // tile
    o = dict(out or {})
    if given is not None:
        o["rice_k"], o["tile_bits"] = given["rice_k"], given["tile_bits"]
    rice_k = o.get("rice_k")
    if rice_k is None:
        rice_k = torch.empty(n_tiles, dtype=torch.uint8, device=dev)
    tile_bits = o.get("tile_bits")
    if tile_bits is None:
        tile_bits = torch.empty(n_tiles, dtype=torch.int32, device=dev)
    total = o.get("total_bits")
    if total is None:
        total = torch.empty(1, dtype=torch.int64, device=dev)
    stream = offs = None
    if pack:
        if capacity_words is None:
            # the optimal k never costs more than k = 8: 4 + coset + 9 n bits
            # (int16 indices: k = 15, 17 n bits)
            per = 17 if idx.dtype == torch.int16 else 9
            capacity_words = n_tiles * ((4 + tile // 2 + per * tile + 31) // 32)
        stream = o.get("stream")
        if stream is None:
            stream = torch.empty(max(int(capacity_words), 1), dtype=torch.int32, device=dev)
        offs = o.get("tile_word_offset")
        if offs is None:
            offs = torch.empty(n_tiles + 1, dtype=torch.int64, device=dev)
    p = make_params(lattice, tile, 4.0,
                    flags=(HQ_RATE_GIVEN if given is not None else 0) | _idx_flag(idx))
    if noalloc:
        # the library's static scratch stands in for the workspace
        ws = None
        code = lib().hq_rate_noalloc(ctypes.byref(p), _ptr(idx), _ptr(coset), n_tiles,
                                     _ptr(rice_k), _ptr(tile_bits), _ptr(total), _ptr(stream),
                                     int(capacity_words or 0), _ptr(offs), _ptr(status),
                                     _stream(dev))
        _check(code, "hq_rate_noalloc")
    else:
        ws = o.get("workspace")
        if ws is None:
            ws = torch.empty(max(rate_workspace_bytes(n_tiles), 8), dtype=torch.uint8, device=dev)
        code = lib().hq_rate(ctypes.byref(p), _ptr(idx), _ptr(coset), n_tiles, _ptr(rice_k),
                             _ptr(tile_bits), _ptr(total), _ptr(stream),
                             int(capacity_words or 0), _ptr(offs), _ptr(ws),
                             0 if ws is None else ws.numel(), _ptr(status), _stream(dev))
        _check(code, "hq_rate")
    res = {"rice_k": rice_k, "tile_bits": tile_bits, "total_bits": total, "workspace": ws}
    if pack:
        res["stream"] = stream
        res["tile_word_offset"] = offs
    return res


class RateItem(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("coset", ctypes.c_void_p), ("n_tiles", ctypes.c_int64),
                ("rice_k", ctypes.c_void_p), ("tile_bits", ctypes.c_void_p),
                ("total_bits", ctypes.c_void_p), ("stream_words", ctypes.c_void_p),
                ("capacity_words", ctypes.c_uint64), ("tile_word_offset", ctypes.c_void_p)]


def hq_rate_batch(encs, lattice="E8", tile=256, pack=False, given=False, status=None,
                  workspace=None, outs=None):
    """hq_rate for several matrices sharing lattice and tile in one call (one
    launch group per eight).  encs: dicts with idx and coset (and, with
    given=True, the encoder's rice_k and tile_bits).  outs: the result of an
    earlier call to write into.  Returns a list of dicts like hq_rate's."""
    if not encs:
        return []
    dev = encs[0]["idx"].device
    items = (RateItem * len(encs))()
    res = []
    for i, e in enumerate(encs):
        _device_tensor(e["idx"], "idx")
        n_tiles = e["idx"].numel() // tile
        o = outs[i] if outs is not None else {}
        rk = e["rice_k"] if given else o.get("rice_k")
        if rk is None:
            rk = torch.empty(n_tiles, dtype=torch.uint8, device=dev)
        tb = e["tile_bits"] if given else o.get("tile_bits")
        if tb is None:
            tb = torch.empty(n_tiles, dtype=torch.int32, device=dev)
        total = o.get("total_bits")
        if total is None:
            total = torch.empty(1, dtype=torch.int64, device=dev)
        r = {"rice_k": rk, "tile_bits": tb, "total_bits": total}
        cap = 0
        if pack:
            per = 17 if e["idx"].dtype == torch.int16 else 9
            cap = n_tiles * ((4 + tile // 2 + per * tile + 31) // 32)
            r["stream"] = o.get("stream")
            if r["stream"] is None:
                r["stream"] = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
            cap = min(cap, r["stream"].numel())
            r["tile_word_offset"] = o.get("tile_word_offset")
            if r["tile_word_offset"] is None:
                r["tile_word_offset"] = torch.empty(n_tiles + 1, dtype=torch.int64, device=dev)
        items[i] = RateItem(_addr(e["idx"]), _addr(e["coset"]), n_tiles, _addr(rk), _addr(tb),
                            _addr(total), _addr(r.get("stream")), cap,
                            _addr(r.get("tile_word_offset")))
        res.append(r)
    nb = lib().hq_rate_batch_workspace_bytes(len(encs), ctypes.byref(items))
    ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                             device=dev)
    p = make_params(lattice, tile, 4.0,
                    flags=(HQ_RATE_GIVEN if given else 0) | _idx_flag(encs[0]["idx"]))
    code = lib().hq_rate_batch(ctypes.byref(p), len(encs), ctypes.byref(items), _ptr(ws),
                               ws.numel(), _ptr(status), _stream(dev))
    _check(code, "hq_rate_batch")
    return res


def _check_packed(stream, offs, lattice, tile, idx, coset, rice_k, idx16, trusted):
    """Host-side checks of an unpack call: the kernel reads the offsets as
    uint64 and the stream words they name on trust, and writes every tile's
    outputs.  Types and sizes are checked first, then device residence;
    unless trusted, the last offset is read back (one 8-byte copy) and
    checked against the stream's length."""
    for t, name in ((stream, "stream"), (offs, "tile_word_offset")):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a tensor" % name)
    if stream.dtype not in (torch.int32, torch.uint32) or stream.dim() != 1:
        raise TypeError("stream must be a 1-D int32 / uint32 tensor of words")
    if offs.dtype != torch.int64 or offs.dim() != 1 or offs.numel() < 1:
        raise TypeError("tile_word_offset must be a 1-D int64 tensor of n_tiles + 1 offsets")
    n_tiles = offs.numel() - 1
    want = torch.int16 if idx16 else torch.int8
    nw = coset_words(lattice, tile)
    if idx is not None and (idx.dtype != want or idx.numel() != n_tiles * tile):
        raise ValueError("idx must hold n_tiles * tile %s values" % str(want).split(".")[-1])
    if coset is not None and nw and (coset.dtype not in (torch.int32, torch.uint32) or
                                     coset.numel() != n_tiles * nw):
        raise ValueError("coset must hold n_tiles * %d int32 words" % nw)
    if rice_k is not None and (rice_k.dtype != torch.uint8 or rice_k.numel() != n_tiles):
        raise ValueError("rice_k must hold n_tiles uint8 values")
    _device_tensor(stream, "stream")
    _device_tensor(offs, "tile_word_offset")
    for t, name in ((idx, "idx"), (coset if nw else None, "coset"), (rice_k, "rice_k")):
        if t is not None:
            _device_tensor(t, name)
    if not trusted and n_tiles > 0:
        last = int(offs[-1].item())
        if last < 0 or last > stream.numel():
            raise ValueError("tile_word_offset[-1] = %d is past the stream's %d words"
                             % (last, stream.numel()))
    return n_tiles


def hq_unpack(stream, tile_word_offset, lattice="E8", tile=256, status=None, out=None,
              idx16=False, trusted=False):
    """Decode a packed stream (as written by hq_rate) back to stripped
    indices (n_tiles, tile) int8 (int16 with idx16), coset words
    (n_tiles, words) int32 or None, and rice_k (n_tiles,) uint8.
    tile_word_offset: int64 (n_tiles + 1).  trusted=True skips the read-back
    of the last offset (for offsets known to fit the stream)."""
    o = dict(out or {})
    n_tiles = _check_packed(stream, tile_word_offset, lattice, tile, o.get("idx"), o.get("coset"),
                            o.get("rice_k"), idx16, trusted)
    dev = stream.device
    idx = o.get("idx")
    if idx is None:
        idx = torch.empty((n_tiles, tile), dtype=torch.int16 if idx16 else torch.int8, device=dev)
    nw = coset_words(lattice, tile)
    coset = o.get("coset")
    if coset is None and nw:
        coset = torch.empty((n_tiles, nw), dtype=torch.int32, device=dev)
    rice_k = o.get("rice_k")
    if rice_k is None:
        rice_k = torch.empty(n_tiles, dtype=torch.uint8, device=dev)
    p = make_params(lattice, tile, 4.0, flags=_idx_flag(idx))
    code = lib().hq_unpack(ctypes.byref(p), _ptr(stream), _ptr(tile_word_offset), n_tiles,
                           _ptr(idx), _ptr(coset if nw else None), _ptr(rice_k), _ptr(status),
                           _stream(dev))
    _check(code, "hq_unpack")
    return {"idx": idx, "coset": coset if nw else None, "rice_k": rice_k}


def _entry_dict(e):
    names = {v: k for k, v in LATTICES.items()}
    return {"name": e.name.decode(), "lattice": names[e.lattice], "tile": e.tile,
            "bps": e.bps, "rht_seed": e.rht_seed, "rows": e.rows, "cols": e.cols,
            "n_tiles": e.n_tiles, "n_words": e.n_words}


def ckpt_save(path, name, packed, scale, rows, cols, lattice="E8", tile=256, bps=4.0,
              rht_seed=0):
    """Append one packed matrix to the checkpoint file `path`: packed is the
    dict hq_rate returns with pack=True (stream, tile_word_offset), scale the
    encode's per-tile scales.  The arrays are copied to host memory."""
    offs = packed["tile_word_offset"].detach().to("cpu", torch.int64).contiguous()
    n_tiles = offs.numel() - 1
    n_words = int(offs[-1])
    if packed["stream"].numel() < n_words:
        raise ValueError("stream holds fewer words than tile_word_offset ends at")
    words = packed["stream"].detach()[:n_words].to("cpu").contiguous()
    sc = scale.detach().to("cpu", torch.float32).contiguous().reshape(-1)
    e = CkptEntry(name.encode(), LATTICES[lattice], tile, bps, rht_seed, rows, cols, n_tiles,
                  n_words)
    _check(lib().hq_ckpt_append(os.fsencode(path), ctypes.byref(e), sc.data_ptr(),
                                offs.data_ptr(), words.data_ptr() if n_words else None),
           "hq_ckpt_append")


def ckpt_entries(path):
    """The entries of a checkpoint file, in file order (list of dicts)."""
    n = ctypes.c_int32()
    _check(lib().hq_ckpt_count(os.fsencode(path), ctypes.byref(n)), "hq_ckpt_count")
    out = []
    for i in range(n.value):
        e = CkptEntry()
        _check(lib().hq_ckpt_entry_at(os.fsencode(path), i, ctypes.byref(e)), "hq_ckpt_entry_at")
        out.append(_entry_dict(e))
    return out


def ckpt_load(path, name, device=None):
    """Read the record `name`: a dict with the entry's fields plus stream
    (int32 words), tile_word_offset (int64) and scale (fp32) on `device`
    (host tensors if None), ready for hq_unpack."""
    meta = {e["name"]: e for e in ckpt_entries(path)}
    if name not in meta:
        raise HQError(HQ_ENOTFOUND, "hq_ckpt_read")
    m = meta[name]
    sc = torch.empty(max(m["n_tiles"], 1), dtype=torch.float32)
    offs = torch.empty(m["n_tiles"] + 1, dtype=torch.int64)
    words = torch.empty(max(m["n_words"], 1), dtype=torch.int32)
    e = CkptEntry()
    _check(lib().hq_ckpt_read(os.fsencode(path), name.encode(), ctypes.byref(e), sc.data_ptr(),
                              offs.data_ptr(), words.data_ptr(), m["n_tiles"], m["n_words"]),
           "hq_ckpt_read")
    res = _entry_dict(e)
    res.update(stream=words, tile_word_offset=offs, scale=sc[:m["n_tiles"]])
    if device is not None:
        for k in ("stream", "tile_word_offset", "scale"):
            res[k] = res[k].to(device)
    return res


class UnpackItem(ctypes.Structure):
    _fields_ = [("stream_words", ctypes.c_void_p), ("tile_word_offset", ctypes.c_void_p),
                ("n_tiles", ctypes.c_int64), ("idx", ctypes.c_void_p),
                ("coset", ctypes.c_void_p), ("rice_k", ctypes.c_void_p)]


def hq_unpack_batch(packs, lattice="E8", tile=256, status=None, outs=None, idx16=False,
                    trusted=False):
    """hq_unpack for several packed matrices sharing lattice and tile, in one
    call (one launch per group of eight).  packs: dicts with "stream" and
    "tile_word_offset" (as hq_rate returns).  Returns a list of dicts like
    hq_unpack's; outs may supply their tensors (int16 indices with idx16).
    The same host-side checks as hq_unpack (trusted: no read-back)."""
    nw = coset_words(lattice, tile)
    res, items = [], []
    dev = None
    for i, pk in enumerate(packs):
        stream, offs = pk["stream"], pk["tile_word_offset"]
        o = dict((outs[i] if outs is not None else None) or {})
        n_tiles = _check_packed(stream, offs, lattice, tile, o.get("idx"), o.get("coset"),
                                o.get("rice_k"), idx16, trusted)
        dev = stream.device
        idx = o.get("idx")
        if idx is None:
            idx = torch.empty((n_tiles, tile), dtype=torch.int16 if idx16 else torch.int8,
                              device=dev)
        elif (idx.dtype == torch.int16) != bool(idx16):
            raise TypeError("outs[%d]['idx'] must be int16 exactly when idx16 is set" % i)
        coset = o.get("coset")
        if coset is None and nw:
            coset = torch.empty((n_tiles, nw), dtype=torch.int32, device=dev)
        rice_k = o.get("rice_k")
        if rice_k is None:
            rice_k = torch.empty(n_tiles, dtype=torch.uint8, device=dev)
        items.append(UnpackItem(stream.data_ptr(), offs.data_ptr(), n_tiles, idx.data_ptr(),
                                coset.data_ptr() if nw else None, rice_k.data_ptr()))
        res.append({"idx": idx, "coset": coset if nw else None, "rice_k": rice_k})
    if not items:
        return res
    arr = (UnpackItem * len(items))(*items)
    p = make_params(lattice, tile, 4.0, flags=HQ_IDX16 if idx16 else 0)
    code = lib().hq_unpack_batch(ctypes.byref(p), len(items), arr, _ptr(status), _stream(dev))
    _check(code, "hq_unpack_batch")
    return res


def hq_gemv(idx, coset, scale, x, rht_seed=0, out=None, workspace=None):
    """y = W x for E8/256-coded weights W (rows, cols) given by idx, coset and
    scale; x: fp32 (cols,) or (m, cols) with m <= 8; returns fp32 (rows,) or
    (m, rows)."""
    for t, name in ((idx, "idx"), (coset, "coset"), (scale, "scale"), (x, "x")):
        _device_tensor(t, name)
    rows, cols = idx.shape
    xv = x.reshape(1, -1) if x.dim() == 1 else x
    m = xv.shape[0]
    dev = idx.device
    y = out if out is not None else torch.empty((m, rows), dtype=torch.float32, device=dev)
    nb = lib().hq_gemv_workspace_bytes(rows, cols, m)
    ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                             device=dev)
    p = make_params("E8", 256, 4.0, rht_seed)
    code = lib().hq_gemv(ctypes.byref(p), _ptr(idx), _ptr(coset), _ptr(scale), rows, cols,
                         _ptr(xv), m, _ptr(y), _ptr(ws), ws.numel(), None, _stream(dev))
    _check(code, "hq_gemv")
    return y.reshape(-1) if x.dim() == 1 else y


def hq_gemm(idx, coset, scale, x, rht_seed=0, out=None, workspace=None):
    """Y = W X^T on the matrix cores for E8/256-coded weights W (rows, cols)
    given by idx, coset and scale; x: fp32 (m, cols), any m >= 1; returns
    fp32 (m, rows)."""
    for t, name in ((idx, "idx"), (coset, "coset"), (scale, "scale"), (x, "x")):
        _device_tensor(t, name)
    rows, cols = idx.shape
    m = x.shape[0]
    dev = idx.device
    y = out if out is not None else torch.empty((m, rows), dtype=torch.float32, device=dev)
    nb = lib().hq_gemm_workspace_bytes(rows, cols, m)
    ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                             device=dev)
    p = make_params("E8", 256, 4.0, rht_seed)
    code = lib().hq_gemm(ctypes.byref(p), _ptr(idx), _ptr(coset), _ptr(scale), rows, cols,
                         _ptr(x), m, _ptr(y), _ptr(ws), ws.numel(), None, _stream(dev))
    _check(code, "hq_gemm")
    return y


def hq_gemv_batch(mats, xs, rht_seed=0, outs=None, workspace=None):
    """hq_gemv for several E8/256-coded matrices in one call: mats is a list
    of dicts with idx, coset and scale, xs the matching fp32 inputs (all 1-D,
    or all (m, cols) with the same m).  Returns the list of outputs."""
    if len(mats) != len(xs):
        raise ValueError("one input per matrix")
    if not mats:
        return []
    dev = mats[0]["idx"].device
    one_d = xs[0].dim() == 1
    m = 1 if one_d else xs[0].shape[0]
    items = (GemvItem * len(mats))()
    ys = []
    for i, (e, x) in enumerate(zip(mats, xs)):
        for name in ("idx", "coset", "scale"):
            _device_tensor(e[name], name)
        _device_tensor(x, "x")
        if (x.dim() == 1) != one_d or (not one_d and x.shape[0] != m):
            raise ValueError("inputs must all be 1-D or all have the same m")
        rows, cols = e["idx"].shape
        y = outs[i] if outs is not None else torch.empty((m, rows), dtype=torch.float32,
                                                          device=dev)
        ys.append(y)
        items[i] = GemvItem(_addr(e["idx"]), _addr(e["coset"]), _addr(e["scale"]), rows, cols,
                            _addr(x), _addr(y))
    nb = lib().hq_gemv_batch_workspace_bytes(len(mats), ctypes.byref(items), m)
    ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                             device=dev)
    p = make_params("E8", 256, 4.0, rht_seed)
    code = lib().hq_gemv_batch(ctypes.byref(p), len(mats), ctypes.byref(items), m, _ptr(ws),
                               ws.numel(), None, _stream(dev))
    _check(code, "hq_gemv_batch")
    return [y.reshape(-1) for y in ys] if one_d else ys


def hq_gemm_batch(mats, xs, rht_seed=0, outs=None, workspace=None):
    """hq_gemm for several E8/256-coded matrices in one call: mats is a list
    of dicts with idx, coset and scale, xs the matching fp32 inputs (m, cols)
    with one m.  Returns the list of fp32 (m, rows) outputs."""
    if len(mats) != len(xs):
        raise ValueError("one input per matrix")
    if not mats:
        return []
    dev = mats[0]["idx"].device
    m = xs[0].shape[0]
    items = (GemvItem * len(mats))()
    ys = []
    for i, (e, x) in enumerate(zip(mats, xs)):
        for name in ("idx", "coset", "scale"):
            _device_tensor(e[name], name)
        _device_tensor(x, "x")
        if x.dim() != 2 or x.shape[0] != m:
            raise ValueError("inputs must all be (m, cols) with the same m")
        rows, cols = e["idx"].shape
        y = outs[i] if outs is not None else torch.empty((m, rows), dtype=torch.float32,
                                                          device=dev)
        ys.append(y)
        items[i] = GemvItem(_addr(e["idx"]), _addr(e["coset"]), _addr(e["scale"]), rows, cols,
                            _addr(x), _addr(y))
    nb = lib().hq_gemm_batch_workspace_bytes(len(mats), ctypes.byref(items), m)
    ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                             device=dev)
    p = make_params("E8", 256, 4.0, rht_seed)
    code = lib().hq_gemm_batch(ctypes.byref(p), len(mats), ctypes.byref(items), m, _ptr(ws),
                               ws.numel(), None, _stream(dev))
    _check(code, "hq_gemm_batch")
    return ys


def hq_kv_scores(q, enc, rht_seed=0, dither_seed=None, dither_base=0, out=None,
                 workspace=None):
    """scores[j][k] = q_j . khat_k for queries q (n_q, 128) fp32 against keys
    encoded by hq_kv_encode (enc: its dict); returns fp32 (n_q, n_keys)."""
    _device_tensor(q, "q")
    idx, coset, scale = enc["idx"], enc["coset"], enc["scale"]
    n_q, n_keys = q.shape[0], idx.shape[0]
    dev = q.device
    sc = out if out is not None else torch.empty((n_q, n_keys), dtype=torch.float32, device=dev)
    nb = lib().hq_kv_scores_workspace_bytes(n_q)
    ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                             device=dev)
    flags = HQ_DITHER if dither_seed is not None else 0
    p = make_params("E8", 128, 4.0, rht_seed, flags,
                    0 if dither_seed is None else dither_seed, dither_base)
    code = lib().hq_kv_scores(ctypes.byref(p), _ptr(q), n_q, _ptr(idx), _ptr(coset), _ptr(scale),
                              n_keys, _ptr(sc), _ptr(ws), ws.numel(), _stream(dev))
    _check(code, "hq_kv_scores")
    return sc


def hq_kv_attention(q, kenc, venc, tau=None, k_cache=None, v_cache=None, out=None,
                    workspace=None):
    """out_hj = softmax_k(tau q_hj . khat_hk) . vhat_h for queries q fp32,
    (n_q, 128) for one head or (n_heads, n_q, 128), over K and V encoded by
    hq_kv_encode for the whole cache (kenc, venc: its dicts; n_heads equal
    runs of keys).  k_cache / v_cache: dicts with the encodes' rht_seed,
    dither_seed (None: rotation-only) and dither_base.  tau defaults to
    1 / sqrt(128).  Returns fp32 shaped like q."""
    _device_tensor(q, "q")
    n_heads = 1 if q.dim() == 2 else q.shape[0]
    n_q = q.shape[-2]
    if kenc["idx"].shape[0] % n_heads:
        raise ValueError("the cache does not split into n_heads equal runs")
    n_keys = kenc["idx"].shape[0] // n_heads
    dev = q.device
    tau = 1.0 / math.sqrt(128.0) if tau is None else tau

    def params(c):
        c = dict(c or {})
        ds = c.get("dither_seed")
        return make_params("E8", 128, 4.0, c.get("rht_seed", 0), HQ_DITHER if ds is not None else 0,
                           0 if ds is None else ds, c.get("dither_base", 0))

    pk, pv = params(k_cache), params(v_cache)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.float32, device=dev)
    nb = lib().hq_kv_attention_workspace_bytes(n_heads, n_q, n_keys)
    ws = workspace if workspace is not None else torch.empty(max(nb, 16), dtype=torch.uint8,
                                                             device=dev)
    code = lib().hq_kv_attention(ctypes.byref(pk), _ptr(kenc["idx"]), _ptr(kenc["coset"]),
                                 _ptr(kenc["scale"]), ctypes.byref(pv), _ptr(venc["idx"]),
                                 _ptr(venc["coset"]), _ptr(venc["scale"]), n_heads, n_keys,
                                 _ptr(q), n_q, tau, _ptr(o), _ptr(ws), ws.numel(), _stream(dev))
    _check(code, "hq_kv_attention")
    return o


def hq_kv_encode(kv, bps=4.0, rht_seed=0, dither_seed=None, dither_base=0, status=None,
                 out=None):
    """Encode KV vectors (n_vectors, head_dim) with E8 and auto scales;
    dither_seed=None gives the rotation-only control."""
    _device_tensor(kv, "kv")
    if kv.dim() != 2:
        raise ValueError("kv must be 2-D (n_vectors, head_dim)")
    n_vec, hd = kv.shape
    dev = kv.device
    o = dict(out or {})
    scale = o.get("scale")
    if scale is None:
        scale = torch.empty(n_vec, dtype=torch.float32, device=dev)
    idx = o.get("idx")
    if idx is None:
        idx = torch.empty((n_vec, hd), dtype=torch.int8, device=dev)
    coset = o.get("coset")
    if coset is None:
        coset = torch.empty((n_vec, coset_words("E8", hd)), dtype=torch.int32, device=dev)
    rice_k = o.get("rice_k")
    if rice_k is None:
        rice_k = torch.empty(n_vec, dtype=torch.uint8, device=dev)
    tile_bits = o.get("tile_bits")
    if tile_bits is None:
        tile_bits = torch.empty(n_vec, dtype=torch.int32, device=dev)
    flags = HQ_SCALE_AUTO | (HQ_DITHER if dither_seed is not None else 0)
    p = make_params("E8", hd, bps, rht_seed, flags,
                    0 if dither_seed is None else dither_seed, dither_base)
    code = lib().hq_kv_encode(ctypes.byref(p), _ptr(kv), _dtype_code(kv.dtype), n_vec,
                              _ptr(scale), _ptr(idx), _ptr(coset), _ptr(rice_k), _ptr(tile_bits),
                              _ptr(status), _stream(dev))
    _check(code, "hq_kv_encode")
    return {"scale": scale, "idx": idx, "coset": coset, "rice_k": rice_k, "tile_bits": tile_bits}


def _addr(t):
    return None if t is None else t.data_ptr()


def _encode_items(xs, lattice, tile, outs):
    """Output dicts (allocated unless given in `outs`) and the C item array
    of a batched encode."""
    dev = xs[0].device
    dt = xs[0].dtype
    res = []
    for i, x in enumerate(xs):
        _device_tensor(x, "x")
        if x.dim() != 2 or x.dtype != dt or x.device != dev:
            raise ValueError("batched matrices must be 2-D with one dtype and device")
        rows, cols = x.shape
        nt = rows * cols // tile if cols % tile == 0 else 0
        o = dict(outs[i]) if outs is not None else {}
        w = max(coset_words(lattice, tile), 1)
        o.setdefault("scale", None)
        res.append({
            "scale": o["scale"] if o["scale"] is not None else
            torch.empty(nt, dtype=torch.float32, device=dev),
            "idx": o.get("idx") if o.get("idx") is not None else
            torch.empty((rows, cols), dtype=torch.int8, device=dev),
            "coset": o.get("coset") if o.get("coset") is not None else
            torch.empty((nt, w), dtype=torch.int32, device=dev),
            "rice_k": o.get("rice_k") if o.get("rice_k") is not None else
            torch.empty(nt, dtype=torch.uint8, device=dev),
            "tile_bits": o.get("tile_bits") if o.get("tile_bits") is not None else
            torch.empty(nt, dtype=torch.int32, device=dev),
        })
    items = (EncodeItem * len(xs))()
    for i, (x, r) in enumerate(zip(xs, res)):
        items[i] = EncodeItem(_addr(x), x.shape[0], x.shape[1], _addr(r["scale"]), _addr(r["idx"]),
                              _addr(r["coset"]), _addr(r["rice_k"]), _addr(r["tile_bits"]))
    return res, items


def _decode_items(encs, out_dtype, outs):
    dev = encs[0]["idx"].device
    ys = []
    items = (DecodeItem * len(encs))()
    for i, e in enumerate(encs):
        _device_tensor(e["idx"], "idx")
        rows, cols = e["idx"].shape
        y = outs[i] if outs is not None else torch.empty((rows, cols), dtype=out_dtype, device=dev)
        if y.dtype != out_dtype:
            raise ValueError("output dtype mismatch")
        ys.append(y)
        items[i] = DecodeItem(_addr(e["idx"]), _addr(e["coset"]), _addr(e["scale"]), rows, cols,
                              _addr(y))
    return ys, items


def hq_encode_batch(xs, lattice="E8", tile=256, bps=4.0, rht_seed=0, outs=None, status=None):
    """hq_encode_tiles on every matrix of `xs` (same dtype, device and
    parameters) in one call; auto scales.  `outs` may give, per matrix, the
    preallocated dict hq_encode_tiles would return.  Returns a list of dicts."""
    if not xs:
        return []
    res, items = _encode_items(xs, lattice, tile, outs)
    p = make_params(lattice, tile, bps, rht_seed, HQ_SCALE_AUTO)
    code = lib().hq_encode_batch(ctypes.byref(p), _dtype_code(xs[0].dtype), len(xs),
                                 ctypes.byref(items), _ptr(status), _stream(xs[0].device))
    _check(code, "hq_encode_batch")
    return res


def hq_decode_batch(encs, lattice="E8", tile=256, rht_seed=0, out_dtype=torch.bfloat16,
                    outs=None, status=None):
    """hq_decode_tiles on every encoded matrix of `encs` (dicts with idx,
    coset, scale) in one call.  Returns the list of decoded tensors."""
    if not encs:
        return []
    ys, items = _decode_items(encs, out_dtype, outs)
    p = make_params(lattice, tile, 4.0, rht_seed, 0)
    code = lib().hq_decode_batch(ctypes.byref(p), _dtype_code(out_dtype), len(encs),
                                 ctypes.byref(items), _ptr(status), _stream(encs[0]["idx"].device))
    _check(code, "hq_decode_batch")
    return ys


def hq_encode_decode_batch(xs, encs, lattice="E8", tile=256, bps=4.0, enc_seed=0, dec_seed=0,
                           out_dtype=torch.bfloat16, enc_outs=None, dec_outs=None, status=None):
    """hq_encode_batch(xs, ..., rht_seed=enc_seed) and hq_decode_batch(encs,
    ..., rht_seed=dec_seed) in one call (one launch on the E8 / tile 256
    path).  `encs` must not share memory with the encode's outputs.
    Returns (encode result dicts, decoded tensors)."""
    if not xs and not encs:
        return [], []
    dev = (xs[0] if xs else encs[0]["idx"]).device
    if xs:
        res, eitems = _encode_items(xs, lattice, tile, enc_outs)
        x_dt = _dtype_code(xs[0].dtype)
    else:
        res, eitems, x_dt = [], None, 1
    if encs:
        ys, ditems = _decode_items(encs, out_dtype, dec_outs)
    else:
        ys, ditems = [], None
    pe = make_params(lattice, tile, bps, enc_seed, HQ_SCALE_AUTO)
    pd = make_params(lattice, tile, 4.0, dec_seed, 0)
    code = lib().hq_encode_decode_batch(
        ctypes.byref(pe), x_dt, len(xs), ctypes.byref(eitems) if eitems is not None else None,
        ctypes.byref(pd), _dtype_code(out_dtype), len(encs),
        ctypes.byref(ditems) if ditems is not None else None, _ptr(status), _stream(dev))
    _check(code, "hq_encode_decode_batch")
    return res, ys
