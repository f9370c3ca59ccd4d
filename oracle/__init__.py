"""CPU oracle of the PlaneZip block codec (ctypes wrapper of ``libpzref.so``).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path (the
HIP library and its binding) must never import it.

The C library follows the PlaneZip paper, §III-A ("Codec" and "Stream format")
and Fig. 2; ``size_model`` is a second, independent implementation of the
candidate sizes, as in the paper's validation (there, an array-based size
calculation was checked against an exact encoder and decoder).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpzref.so")
# A sanitizer build of the same source may be substituted (tests only).
_LIB_PATH = os.environ.get("PZREF_LIB", _LIB_PATH)

ZVC, DBX, BX, ZBX, RAW = 0, 1, 2, 3, 4
CANDIDATES = ("ZVC", "DBX", "BX", "ZBX", "RAW")
ALL_CODECS = 0x1F
OK, EINVAL, ENOSPC, ECORRUPT = 0, 1, 2, 3

BLOCK_BYTES = 128
CHUNK_BYTES = 4096


def _load():
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u64p = ctypes.POINTER(ctypes.c_uint64)
    sz = ctypes.c_size_t
    sig = {
        "pzref_width": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
        "pzref_num_chunks": (sz, [sz]),
        "pzref_max_compressed": (sz, [sz]),
        "pzref_encode_candidate": (ctypes.c_int, [u8p, ctypes.c_int, ctypes.c_int, u8p, sz, i64p]),
        "pzref_decode_candidate": (ctypes.c_int, [u8p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, u8p, i64p]),
        "pzref_block_sizes": (ctypes.c_int, [u8p, ctypes.c_int, i32p]),
        "pzref_code_planes": (ctypes.c_int, [u64p, ctypes.c_int, ctypes.c_int, ctypes.c_int, u8p, sz, i64p]),
        "pzref_decode_planes": (ctypes.c_int, [u8p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, u64p, i64p]),
        "pzref_compress_chunk": (ctypes.c_int64, [u8p, sz, ctypes.c_int, ctypes.c_uint32, ctypes.c_int, u8p, u8p, i32p]),
        "pzref_compress": (ctypes.c_int64, [u8p, sz, ctypes.c_int, ctypes.c_uint32, ctypes.c_int, u8p, sz, u8p, i32p]),
        "pzref_decompress": (ctypes.c_int, [u8p, sz, ctypes.c_int, ctypes.c_uint32, ctypes.c_int, u8p, sz]),
        "pzref_compress_mt": (ctypes.c_int64, [u8p, sz, ctypes.c_int, ctypes.c_uint32, ctypes.c_int, u8p, sz, ctypes.c_int]),
        "pzref_decompress_mt": (ctypes.c_int, [u8p, sz, ctypes.c_int, ctypes.c_uint32, ctypes.c_int, u8p, sz, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _u8(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _as_bytes(x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    return a.view(np.uint8).reshape(-1)


def width(dtype: int, elem_bits: int) -> int:
    return lib().pzref_width(dtype, elem_bits)


def num_chunks(raw_bytes: int) -> int:
    return (raw_bytes + CHUNK_BYTES - 1) // CHUNK_BYTES


def max_compressed(raw_bytes: int) -> int:
    return 2 * num_chunks(raw_bytes) + raw_bytes


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle error {code}")
        self.code = code


def compress(data, w: int, codec_mask: int = ALL_CODECS, tagged: bool = True,
             want_blocks: bool = False, threads: int = 1):
    """Compress a tensor's bytes. Returns the stream (uint8 array), or
    (stream, tags, block_bits) with ``want_blocks``."""
    src = _as_bytes(data)
    n = src.size
    cap = max_compressed(n)
    dst = np.zeros(max(cap, 1), dtype=np.uint8)
    nblocks = num_chunks(n) * 32
    if want_blocks:
        tags = np.zeros(max(nblocks, 1), dtype=np.uint8)
        bits = np.zeros(max(nblocks, 1), dtype=np.int32)
        r = lib().pzref_compress(_u8(src), n, w, codec_mask, int(tagged), _u8(dst), cap,
                                 _u8(tags), bits.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    elif threads > 1:
        r = lib().pzref_compress_mt(_u8(src), n, w, codec_mask, int(tagged), _u8(dst), cap, threads)
    else:
        r = lib().pzref_compress(_u8(src), n, w, codec_mask, int(tagged), _u8(dst), cap, None, None)
    if r < 0:
        raise OracleError(-r, "compress")
    out = dst[:r].copy()
    if want_blocks:
        nb = (n + BLOCK_BYTES - 1) // BLOCK_BYTES
        # Blocks are numbered 32 per chunk; the tail chunk may hold fewer.
        idx = _block_index(n)
        assert idx.size == nb
        return out, tags[idx].copy(), bits[idx].copy()
    return out


def _block_index(raw_bytes: int) -> np.ndarray:
    """Per-chunk block slots (32 per chunk) that hold real blocks, in order."""
    nb = (raw_bytes + BLOCK_BYTES - 1) // BLOCK_BYTES
    return np.arange(nb, dtype=np.int64)


def compress_chunk(data, w: int, codec_mask: int = ALL_CODECS, tagged: bool = True):
    """One chunk (1..4096 bytes). Returns (H, payload bytes, tags, block_bits)."""
    src = _as_bytes(data)
    n = src.size
    payload = np.zeros(max(n, 1), dtype=np.uint8)
    tags = np.zeros(32, dtype=np.uint8)
    bits = np.zeros(32, dtype=np.int32)
    r = lib().pzref_compress_chunk(_u8(src), n, w, codec_mask, int(tagged), _u8(payload),
                                   _u8(tags), bits.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if r < 0:
        raise OracleError(-r, "compress_chunk")
    nb = (n + BLOCK_BYTES - 1) // BLOCK_BYTES
    return int(r), payload[:r].copy(), tags[:nb].copy(), bits[:nb].copy()


def decompress(stream, raw_bytes: int, w: int, codec_mask: int = ALL_CODECS,
               tagged: bool = True, threads: int = 1) -> np.ndarray:
    """Decode a stream; raises OracleError on a corrupt stream."""
    src = _as_bytes(stream)
    dst = np.zeros(max(raw_bytes, 1), dtype=np.uint8)
    if threads > 1:
        rc = lib().pzref_decompress_mt(_u8(src), src.size, w, codec_mask, int(tagged), _u8(dst),
                                       raw_bytes, threads)
    else:
        rc = lib().pzref_decompress(_u8(src), src.size, w, codec_mask, int(tagged), _u8(dst), raw_bytes)
    if rc != OK:
        raise OracleError(rc, "decompress")
    return dst[:raw_bytes]


def decompress_status(stream, raw_bytes: int, w: int, codec_mask: int = ALL_CODECS,
                      tagged: bool = True) -> int:
    """Status code of decoding a stream (OK or ECORRUPT)."""
    src = _as_bytes(stream)
    dst = np.zeros(max(raw_bytes, 1), dtype=np.uint8)
    return lib().pzref_decompress(_u8(src), src.size, w, codec_mask, int(tagged), _u8(dst), raw_bytes)


def block_sizes(block, w: int) -> np.ndarray:
    """Bit counts of the five candidates of one 128-byte block."""
    b = _as_bytes(block)
    assert b.size == BLOCK_BYTES
    out = np.zeros(5, dtype=np.int32)
    rc = lib().pzref_block_sizes(_u8(b), w, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != OK:
        raise OracleError(rc, "block_sizes")
    return out


def blocks_sizes(blocks, w: int) -> np.ndarray:
    """Candidate bit counts of many blocks: (nblocks, 5)."""
    b = _as_bytes(blocks).reshape(-1, BLOCK_BYTES)
    out = np.zeros((b.shape[0], 5), dtype=np.int32)
    fn = lib().pzref_block_sizes
    i32p = ctypes.POINTER(ctypes.c_int32)
    base = b.ctypes.data
    obase = out.ctypes.data
    for i in range(b.shape[0]):
        rc = fn(ctypes.cast(base + i * BLOCK_BYTES, ctypes.POINTER(ctypes.c_uint8)), w,
                ctypes.cast(obase + i * 20, i32p))
        if rc != OK:
            raise OracleError(rc, "block_sizes")
    return out


def encode_candidate(block, w: int, cand: int):
    """Payload bytes and bit count of one candidate of one block."""
    b = _as_bytes(block)
    out = np.zeros(256, dtype=np.uint8)
    nbits = ctypes.c_int64(0)
    rc = lib().pzref_encode_candidate(_u8(b), w, cand, _u8(out), out.size, ctypes.byref(nbits))
    if rc != OK:
        raise OracleError(rc, "encode_candidate")
    return out[: (nbits.value + 7) // 8].copy(), nbits.value


def decode_candidate(payload, nbits: int, w: int, cand: int):
    """Decoded 128-byte block and bits consumed; raises on a corrupt payload."""
    src = _as_bytes(payload)
    if src.size == 0:
        src = np.zeros(1, dtype=np.uint8)
    out = np.zeros(BLOCK_BYTES, dtype=np.uint8)
    used = ctypes.c_int64(0)
    rc = lib().pzref_decode_candidate(_u8(src), nbits, w, cand, _u8(out), ctypes.byref(used))
    if rc != OK:
        raise OracleError(rc, "decode_candidate")
    return out, used.value


def code_planes(planes, K: int, L: int, R: int):
    """Plane coder alone: returns (bytes, nbits)."""
    P = np.ascontiguousarray(np.asarray(planes, dtype=np.uint64).reshape(-1))
    assert P.size == K
    out = np.zeros(512, dtype=np.uint8)
    nbits = ctypes.c_int64(0)
    rc = lib().pzref_code_planes(P.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), K, L, R,
                                 _u8(out), out.size, ctypes.byref(nbits))
    if rc != OK:
        raise OracleError(rc, "code_planes")
    return out[: (nbits.value + 7) // 8].copy(), nbits.value


def decode_planes(payload, nbits: int, K: int, L: int, R: int):
    """Inverse of code_planes: returns (planes, bits consumed)."""
    src = _as_bytes(payload)
    if src.size == 0:
        src = np.zeros(1, dtype=np.uint8)
    P = np.zeros(K, dtype=np.uint64)
    used = ctypes.c_int64(0)
    rc = lib().pzref_decode_planes(_u8(src), nbits, K, L, R,
                                   P.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), ctypes.byref(used))
    if rc != OK:
        raise OracleError(rc, "decode_planes")
    return P, used.value


def header_table(stream, raw_bytes: int) -> np.ndarray:
    """The u16 header values H[0..C-1] of a stream (no validation)."""
    C = num_chunks(raw_bytes)
    return _as_bytes(stream)[: 2 * C].view("<u2").astype(np.int64)


def sampled_size(data, w: int, stride: int, threads: int = 1):
    """The size measurement over chunks 0, stride, 2*stride, ... of a tensor
    (the paper's methodology compresses tensors above 32 MB on every fourth
    4 KB chunk, §IV "Tensor capture"): the whole tensor is compressed and the
    sampled chunks' stream bytes (2 + H each), raw bytes and header values are
    read off its header table. Returns (stream bytes, raw bytes, H values)."""
    src = _as_bytes(data)
    n = src.size
    H = header_table(compress(src, w, threads=threads), n)
    picked = np.arange(0, num_chunks(n), stride, dtype=np.int64)
    raw = np.minimum(CHUNK_BYTES, n - picked * CHUNK_BYTES)
    return int((2 + H[picked]).sum()), int(raw.sum()), H[picked]
