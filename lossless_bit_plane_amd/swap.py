"""Swap engine and saved-tensor hooks (the ``pz_swap*`` calls of the C ABI;
the copy path of the PlaneZip paper, §III and Fig. 2).

Argument marshalling only: the pool, the staging slots, the copies and the
worker thread live in the native library. ``SwapHooks`` routes the tensors
that autograd saves for the backward pass through it.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import PZ_ERROR_CORRUPT_STREAM, PlaneZipError, check, lib
from .codec import _TORCH_DTYPE, OTHER, _byte_view, _stream


class Swapper:
    """One engine: a pinned pool of ``pool_chunks`` chunks of
    ``pool_chunk_bytes`` and ``staging_slots`` device staging buffers of
    ``staging_bytes`` (the largest tensor it takes is about that size)."""

    def __init__(self, pool_chunk_bytes: int, pool_chunks: int, staging_bytes: int, staging_slots: int = 4):
        self.handle = lib.pz_swapper_create(pool_chunk_bytes, pool_chunks, staging_bytes, staging_slots)
        if not self.handle:
            raise RuntimeError("pz_swapper_create failed (bad sizes, no device or out of memory)")
        self.pool_chunk_bytes = pool_chunk_bytes
        self.staging_bytes = staging_bytes
        self._raw = {}  # ticket -> raw bytes, to check swap-in destinations

    def close(self) -> None:
        h, self.handle = getattr(self, "handle", None), None
        if h:
            lib.pz_swapper_destroy(h)

    __del__ = close

    def free_chunks(self) -> int:
        return int(lib.pz_swapper_free_chunks(self.handle))

    def swap_out(self, src: torch.Tensor, dtype=None, elem_bits=None, stream=None) -> int:
        """pz_swap_out: returns the ticket."""
        if dtype is None:
            dtype, bits = _TORCH_DTYPE.get(src.dtype, (OTHER, 32))
            elem_bits = bits if elem_bits is None else elem_bits
        b = _byte_view(src)
        ticket = ctypes.c_uint64(0)
        check(lib.pz_swap_out(self.handle, b.data_ptr(), b.numel(), dtype, 32 if elem_bits is None else elem_bits,
                              _stream(stream), ctypes.byref(ticket)), "pz_swap_out")
        self._raw[int(ticket.value)] = b.numel()
        return int(ticket.value)

    def wait(self, ticket: int) -> int:
        """pz_swap_wait: the stream's length once it is in the pool."""
        n = ctypes.c_uint64(0)
        check(lib.pz_swap_wait(self.handle, ticket, ctypes.byref(n)), "pz_swap_wait")
        return int(n.value)

    def swap_in(self, ticket: int, dst: torch.Tensor, status: torch.Tensor | None = None, stream=None):
        """pz_swap_in into ``dst`` (contiguous, the swapped-out size)."""
        b = _byte_view(dst)
        if b.numel() < self._raw.get(ticket, 0):
            raise ValueError(f"swap-in destination holds {b.numel()} bytes, the tensor {self._raw[ticket]}")
        check(lib.pz_swap_in(self.handle, ticket, b.data_ptr(), status.data_ptr() if status is not None else None,
                             _stream(stream)), "pz_swap_in")
        return dst

    def release(self, ticket: int) -> None:
        check(lib.pz_swap_release(self.handle, ticket), "pz_swap_release")
        self._raw.pop(ticket, None)

    def read(self, ticket: int):
        """pz_swap_read: the ticket's stream as a numpy uint8 array."""
        import numpy as np

        n = self.wait(ticket)
        out = np.empty(max(n, 1), dtype=np.uint8)
        got = ctypes.c_uint64(0)
        check(lib.pz_swap_read(self.handle, ticket, out.ctypes.data, out.size, ctypes.byref(got)), "pz_swap_read")
        return out[: got.value]


class SwapHooks:
    """Context manager: inside it, every tensor autograd saves that is a
    contiguous CUDA BF16 or FP32 tensor of at least ``min_bytes`` goes through
    the swapper when saved (compressed, copied to the pinned pool, its device
    memory left to the caching allocator) and comes back when the backward
    pass unpacks it (copied in, decompressed). ``check`` synchronizes after
    each swap-in and raises on a corrupt stream."""

    def __init__(self, swapper: Swapper, min_bytes: int = 1 << 20, check: bool = False):
        self.swapper = swapper
        self.min_bytes = min_bytes
        self.check = check
        self.swapped = 0
        self.swapped_bytes = 0
        self._ctx = torch.autograd.graph.saved_tensors_hooks(self._pack, self._unpack)

    def __enter__(self):
        self._ctx.__enter__()
        return self

    def __exit__(self, *exc):
        return self._ctx.__exit__(*exc)

    def _pack(self, t: torch.Tensor):
        nbytes = t.numel() * t.element_size()
        if (not t.is_cuda or t.dtype not in _TORCH_DTYPE or not t.is_contiguous() or nbytes < self.min_bytes
                or nbytes + 2 * ((nbytes + 4095) // 4096) > self.swapper.staging_bytes):
            return t
        ticket = self.swapper.swap_out(t)
        self.swapped += 1
        self.swapped_bytes += nbytes
        return (_Swapped(self.swapper, ticket), t.shape, t.dtype, t.device, t.requires_grad)

    def _unpack(self, packed):
        if isinstance(packed, torch.Tensor):
            return packed
        handle, shape, dtype, device, _ = packed
        out = torch.empty(shape, dtype=dtype, device=device)
        status = torch.zeros(1, dtype=torch.int32, device=device) if self.check else None
        self.swapper.swap_in(handle.ticket, out, status)
        if self.check and int(status.item()) != 0:
            raise PlaneZipError(PZ_ERROR_CORRUPT_STREAM, "pz_swap_in (device status)")
        return out


class _Swapped:
    """A ticket that returns its pool chunks when autograd drops the packed
    value (after the backward pass, or with the graph)."""

    def __init__(self, swapper: Swapper, ticket: int):
        self.swapper = swapper
        self.ticket = ticket

    def __del__(self):
        if self.swapper.handle:
            lib.pz_swap_release(self.swapper.handle, self.ticket)
            self.swapper._raw.pop(self.ticket, None)
