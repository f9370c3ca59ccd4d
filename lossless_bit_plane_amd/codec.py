"""Python entry points with the names of the C ABI (argument marshalling only).

Tensors must be contiguous device tensors; the stream defaults to the current
torch stream. Every call only enqueues work, like the C functions (except
with the PZ_DEBUG environment variable set, when pz_compressed_size also
prints the size pass's per-block tags and sizes and synchronizes).
"""
from __future__ import annotations

import ctypes
import os
import sys

import torch

from ._lib import PZ_ERROR_CORRUPT_STREAM, PlaneZipError, check, lib

BF16, FP32, OTHER = 0, 1, 2
# Candidate masks of the codec-variant calls (bit t allows tag t).
CODEC_ZVC, CODEC_DBX, CODEC_BX, CODEC_ZBX, CODEC_RAW = 1, 2, 4, 8, 16
CODEC_ALL = 0x1F
_TORCH_DTYPE = {torch.bfloat16: (BF16, 16), torch.float32: (FP32, 32)}


def num_chunks(raw_bytes: int) -> int:
    return (raw_bytes + 4095) // 4096


def max_compressed_bytes(raw_bytes: int) -> int:
    return 2 * num_chunks(raw_bytes) + raw_bytes


def _stream_obj(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream):
    return _stream_obj(stream).cuda_stream


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _byte_view(t: torch.Tensor) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError("PlaneZip works on device tensors only")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.reshape(-1).view(torch.uint8)


def _kind(t: torch.Tensor, dtype, elem_bits):
    if dtype is None:
        dtype, bits = _TORCH_DTYPE.get(t.dtype, (OTHER, 32))
        elem_bits = bits if elem_bits is None else elem_bits
    return dtype, (32 if elem_bits is None else elem_bits)


def pz_compressed_size(src: torch.Tensor, dtype=None, elem_bits=None, chunk_lens: bool = False,
                       stream=None):
    """Device int64 tensor (1,) with the exact stream size, and optionally the
    int16 (bit pattern of uint16) chunk header values."""
    dtype, elem_bits = _kind(src, dtype, elem_bits)
    b = _byte_view(src)
    out = torch.empty(1, dtype=torch.int64, device=b.device)
    lens = torch.empty(num_chunks(b.numel()), dtype=torch.int16, device=b.device) if chunk_lens else None
    check(lib.pz_compressed_size(_ptr(b), b.numel(), dtype, elem_bits, _ptr(out), _ptr(lens),
                                 _stream(stream)), "pz_compressed_size")
    if os.environ.get("PZ_DEBUG"):
        _debug_dump(src, dtype, elem_bits, out, stream)
    return out, lens


_TAG_NAMES = ("ZVC", "DBX", "BX", "ZBX", "RAW")


def _debug_dump(src, dtype, elem_bits, out, stream):
    """PZ_DEBUG=1: the size pass's per-block tags (a histogram) and the mean
    size of every candidate, on stderr; PZ_DEBUG=2: also one line per block
    (tag and the five candidate sizes in bits). Synchronizes the stream."""
    sizes, tags = pz_block_sizes(src, dtype, elem_bits, stream=stream)
    s = _stream_obj(stream)
    s.synchronize()
    sz = sizes.cpu().view(torch.uint16).to(torch.int64) if sizes.numel() else torch.zeros((0, 5), dtype=torch.int64)
    tg = tags.cpu().to(torch.int64)
    nb = tg.numel()
    hist = torch.bincount(tg, minlength=5).tolist() if nb else [0] * 5
    mean = (sz.double().mean(dim=0).tolist() if nb else [0.0] * 5)
    print(f"[PZ_DEBUG] {nb} blocks, w={elem_bits}, stream {int(out.item())} bytes; tags "
          + ", ".join(f"{n} {c}" for n, c in zip(_TAG_NAMES, hist))
          + "; mean candidate bits " + ", ".join(f"{n} {m:.1f}" for n, m in zip(_TAG_NAMES, mean)),
          file=sys.stderr, flush=True)
    if os.environ.get("PZ_DEBUG") == "2":
        for i in range(nb):
            print(f"[PZ_DEBUG] block {i}: {_TAG_NAMES[int(tg[i])]} "
                  + " ".join(str(int(v)) for v in sz[i].tolist()), file=sys.stderr)


def pz_compressed_size_sampled(src: torch.Tensor, chunk_stride: int = 4, dtype=None, elem_bits=None,
                               chunk_lens: bool = False, stream=None):
    """Device int64 tensor (2,): the stream bytes of chunks 0, stride,
    2*stride, ... and their raw bytes; optionally their int16 (bit pattern of
    uint16) header values."""
    dtype, elem_bits = _kind(src, dtype, elem_bits)
    b = _byte_view(src)
    out = torch.empty(2, dtype=torch.int64, device=b.device)
    n = (num_chunks(b.numel()) + chunk_stride - 1) // chunk_stride if chunk_stride > 0 else 0
    lens = torch.empty(max(n, 1), dtype=torch.int16, device=b.device) if chunk_lens else None
    check(lib.pz_compressed_size_sampled(_ptr(b), b.numel(), dtype, elem_bits, chunk_stride, _ptr(out),
                                         _ptr(lens), _stream(stream)), "pz_compressed_size_sampled")
    return out, (lens[:n] if lens is not None else None)


def pz_block_sizes(src: torch.Tensor, dtype=None, elem_bits=None, stream=None):
    """Per-block candidate sizes (int16 view of uint16, shape (nblocks, 5))
    and chosen tags (uint8, nblocks)."""
    dtype, elem_bits = _kind(src, dtype, elem_bits)
    b = _byte_view(src)
    nb = (b.numel() + 127) // 128
    sizes = torch.empty((max(nb, 1), 5), dtype=torch.int16, device=b.device)
    tags = torch.empty(max(nb, 1), dtype=torch.uint8, device=b.device)
    check(lib.pz_block_sizes(_ptr(b), b.numel(), dtype, elem_bits, _ptr(sizes), _ptr(tags),
                             _stream(stream)), "pz_block_sizes")
    return sizes[:nb], tags[:nb]


def pz_compress(src: torch.Tensor, dtype=None, elem_bits=None, dst: torch.Tensor | None = None,
                out_bytes: torch.Tensor | None = None, stream=None):
    """Compress into ``dst`` (uint8, capacity >= max_compressed_bytes).
    Returns (dst, out_bytes) where out_bytes is a device int64 tensor (1,)."""
    dtype, elem_bits = _kind(src, dtype, elem_bits)
    b = _byte_view(src)
    cap = max_compressed_bytes(b.numel())
    if dst is None:
        dst = torch.empty(max(cap, 16), dtype=torch.uint8, device=b.device)
    if out_bytes is None:
        out_bytes = torch.empty(1, dtype=torch.int64, device=b.device)
    check(lib.pz_compress(_ptr(b), b.numel(), dtype, elem_bits, _ptr(dst), dst.numel(),
                          _ptr(out_bytes), _stream(stream)), "pz_compress")
    return dst, out_bytes


def pz_compress_noalloc(src: torch.Tensor, dst: torch.Tensor, out_bytes: torch.Tensor, dtype=None,
                        elem_bits=None, stream=None):
    """pz_compress into caller-provided ``dst`` (uint8, capacity >=
    max_compressed_bytes) and ``out_bytes`` (int64, 1) through the entry
    point that allocates nothing (tensors up to PZ_NOALLOC_MAX_BYTES; calls
    that overlap on one GPU race). Returns (dst, out_bytes)."""
    dtype, elem_bits = _kind(src, dtype, elem_bits)
    b = _byte_view(src)
    check(lib.pz_compress_noalloc(_ptr(b), b.numel(), dtype, elem_bits, _ptr(dst), dst.numel(),
                                  _ptr(out_bytes), _stream(stream)), "pz_compress_noalloc")
    return dst, out_bytes


def pz_decompress(src: torch.Tensor, comp_bytes: int, raw_bytes: int, dtype: int, elem_bits: int,
                  dst: torch.Tensor | None = None, status: torch.Tensor | None = None, stream=None):
    """Decompress ``comp_bytes`` of ``src`` into ``dst`` (uint8, raw_bytes).
    Returns (dst, status) where status is a device int32 tensor (1,)."""
    b = _byte_view(src)
    if dst is None:
        dst = torch.empty(max(raw_bytes, 16), dtype=torch.uint8, device=b.device)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=b.device)
    check(lib.pz_decompress(_ptr(b), comp_bytes, dtype, elem_bits, _ptr(dst), raw_bytes,
                            _ptr(status), _stream(stream)), "pz_decompress")
    return dst, status


def pz_compressed_size_ex(src: torch.Tensor, codec_mask: int, tagged: bool, dtype=None,
                          elem_bits=None, chunk_lens: bool = False, stream=None):
    """pz_compressed_size for a codec variant (candidate mask, tagged or not)."""
    dtype, elem_bits = _kind(src, dtype, elem_bits)
    b = _byte_view(src)
    out = torch.empty(1, dtype=torch.int64, device=b.device)
    lens = torch.empty(num_chunks(b.numel()), dtype=torch.int16, device=b.device) if chunk_lens else None
    check(lib.pz_compressed_size_ex(_ptr(b), b.numel(), dtype, elem_bits, codec_mask, int(tagged),
                                    _ptr(out), _ptr(lens), _stream(stream)), "pz_compressed_size_ex")
    return out, lens


def pz_compress_ex(src: torch.Tensor, codec_mask: int, tagged: bool, dtype=None, elem_bits=None,
                   dst: torch.Tensor | None = None, out_bytes: torch.Tensor | None = None,
                   stream=None):
    """pz_compress for a codec variant (candidate mask, tagged or not)."""
    dtype, elem_bits = _kind(src, dtype, elem_bits)
    b = _byte_view(src)
    cap = max_compressed_bytes(b.numel())
    if dst is None:
        dst = torch.empty(max(cap, 16), dtype=torch.uint8, device=b.device)
    if out_bytes is None:
        out_bytes = torch.empty(1, dtype=torch.int64, device=b.device)
    check(lib.pz_compress_ex(_ptr(b), b.numel(), dtype, elem_bits, codec_mask, int(tagged), _ptr(dst),
                             dst.numel(), _ptr(out_bytes), _stream(stream)), "pz_compress_ex")
    return dst, out_bytes


def pz_decompress_ex(src: torch.Tensor, comp_bytes: int, raw_bytes: int, dtype: int, elem_bits: int,
                     codec_mask: int, tagged: bool, dst: torch.Tensor | None = None,
                     status: torch.Tensor | None = None, stream=None):
    """pz_decompress for a stream written by pz_compress_ex with the same
    (codec_mask, tagged)."""
    b = _byte_view(src)
    if dst is None:
        dst = torch.empty(max(raw_bytes, 16), dtype=torch.uint8, device=b.device)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=b.device)
    check(lib.pz_decompress_ex(_ptr(b), comp_bytes, dtype, elem_bits, codec_mask, int(tagged),
                               _ptr(dst), raw_bytes, _ptr(status), _stream(stream)), "pz_decompress_ex")
    return dst, status


def _ptr_array(ts):
    return (ctypes.c_void_p * max(1, len(ts)))(*[_ptr(t) for t in ts])


def _size_array(vals):
    return (ctypes.c_size_t * max(1, len(vals)))(*[int(v) for v in vals])


def pz_compress_batch(srcs, dtype: int, elem_bits: int, dsts=None, out_bytes: torch.Tensor | None = None,
                      stream=None):
    """pz_compress on several tensors of one (dtype, elem_bits) in as few
    launches as possible. Returns (dsts, out_bytes): a list of uint8 streams
    (capacity max_compressed_bytes each) and a device int64 tensor (n,)."""
    bs = [_byte_view(t) for t in srcs]
    if not bs:
        raise ValueError("pz_compress_batch: no tensors")
    dev = bs[0].device
    if dsts is None:
        dsts = [torch.empty(max(max_compressed_bytes(b.numel()), 16), dtype=torch.uint8, device=dev) for b in bs]
    if out_bytes is None:
        out_bytes = torch.empty(len(bs), dtype=torch.int64, device=dev)
    check(lib.pz_compress_batch(len(bs), _ptr_array(bs), _size_array([b.numel() for b in bs]), dtype, elem_bits,
                                _ptr_array(dsts), _size_array([d.numel() for d in dsts]), _ptr(out_bytes),
                                _stream(stream)), "pz_compress_batch")
    return dsts, out_bytes


def pz_compressed_size_batch(srcs, dtype: int, elem_bits: int, chunk_lens: bool = False, stream=None):
    """pz_compressed_size on several tensors of one (dtype, elem_bits) in as
    few launches as possible. Returns (out_bytes, lens): a device int64
    tensor (n,) and, with chunk_lens, a list of int16 header tensors."""
    bs = [_byte_view(t) for t in srcs]
    if not bs:
        raise ValueError("pz_compressed_size_batch: no tensors")
    dev = bs[0].device
    out = torch.empty(len(bs), dtype=torch.int64, device=dev)
    lens = [torch.empty(max(1, num_chunks(b.numel())), dtype=torch.int16, device=dev) for b in bs] if chunk_lens else None
    check(lib.pz_compressed_size_batch(len(bs), _ptr_array(bs), _size_array([b.numel() for b in bs]), dtype,
                                       elem_bits, _ptr(out), _ptr_array(lens) if lens else None, _stream(stream)),
          "pz_compressed_size_batch")
    if lens is not None:
        lens = [ln[: num_chunks(b.numel())] for ln, b in zip(lens, bs)]
    return out, lens


def pz_decompress_batch(srcs, comp_bytes, raw_bytes, dtype: int, elem_bits: int, dsts=None,
                        status: torch.Tensor | None = None, stream=None):
    """pz_decompress on several streams of one (dtype, elem_bits). Returns
    (dsts, status): a list of uint8 tensors (raw_bytes each) and a device
    int32 tensor (n,)."""
    bs = [_byte_view(t) for t in srcs]
    if not bs or len(comp_bytes) != len(bs) or len(raw_bytes) != len(bs):
        raise ValueError("pz_decompress_batch: one comp_bytes and raw_bytes per stream")
    dev = bs[0].device
    if dsts is None:
        dsts = [torch.empty(max(int(r), 16), dtype=torch.uint8, device=dev) for r in raw_bytes]
    if status is None:
        status = torch.empty(len(bs), dtype=torch.int32, device=dev)
    check(lib.pz_decompress_batch(len(bs), _ptr_array(bs), _size_array(comp_bytes), dtype, elem_bits,
                                  _ptr_array(dsts), _size_array(raw_bytes), _ptr(status), _stream(stream)),
          "pz_decompress_batch")
    return dsts, status


def compress(t: torch.Tensor, dtype=None, elem_bits=None):
    """Compress and synchronize: returns the stream as a uint8 device tensor
    of its exact length."""
    dst, nbytes = pz_compress(t, dtype, elem_bits)
    n = int(nbytes.item())
    return dst[:n]


def decompress(stream_bytes: torch.Tensor, raw_bytes: int, dtype: int, elem_bits: int):
    """Decompress and synchronize; raises on a corrupt stream. Returns uint8."""
    dst, status = pz_decompress(stream_bytes, stream_bytes.numel(), raw_bytes, dtype, elem_bits)
    st = int(status.item())
    if st != 0:
        raise PlaneZipError(PZ_ERROR_CORRUPT_STREAM if st == PZ_ERROR_CORRUPT_STREAM else st,
                            "pz_decompress (device status)")
    return dst[:raw_bytes]
