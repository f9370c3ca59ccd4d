"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every function declared in include/planezip.h, and rejects bad arguments
synchronously before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^\s*(?:pz_status_t|const char \*|pz_predictor_t \*|pz_swapper_t \*|void|size_t|double)\s*(pz_\w+)\s*\(",
                                text, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    path = os.path.join(ROOT, "lossless_bit_plane_amd", "libplanezip.so")
    if not os.path.exists(path):
        pytest.fail("libplanezip.so is not built (run __graft_entry__.build())")
    from lossless_bit_plane_amd import _lib

    return _lib.lib


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) >= {"pz_compress", "pz_decompress", "pz_compressed_size"}
    assert {"pz_compressed_size_sampled", "pz_predictor_create", "pz_predictor_update",
            "pz_predictor_predict", "pz_predictor_destroy"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), name
    from lossless_bit_plane_amd import _lib

    assert set(_lib.EXPORTS) == set(declared)


def test_rejects_bad_arguments_on_host(lib):
    from lossless_bit_plane_amd import _lib

    vp = ctypes.c_void_p
    fake = 256  # aligned, never dereferenced: every call below fails its checks first
    # Unsupported (dtype, elem_bits) pairs.
    assert lib.pz_compress(fake, 100, 0, 8, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress(fake, 100, 1, 16, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress(fake, 100, 3, 32, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    # Null pointers with data.
    assert lib.pz_compress(None, 100, 0, 16, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress(fake, 100, 0, 16, fake, 1000, None, None) == _lib.PZ_ERROR_INVALID_VALUE
    # Misaligned source.
    assert lib.pz_compress(fake + 4, 100, 0, 16, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    # Capacity below the worst case 2*chunks + raw.
    assert lib.pz_compress(fake, 4097, 0, 16, fake, 4100, fake, None) == _lib.PZ_ERROR_INSUFFICIENT_BUFFER
    # A stream shorter than its header table.
    assert lib.pz_decompress(fake, 3, 0, 16, fake, 8193, None, None) == _lib.PZ_ERROR_CORRUPT_STREAM
    assert lib.pz_compressed_size(fake, 10, 2, 16, fake, None, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_status_string(3) == b"corrupt stream"


def test_rejects_bad_codec_modes_on_host(lib):
    from lossless_bit_plane_amd import _lib

    fake = 256  # aligned, never dereferenced: every call below fails its checks first
    bad = _lib.PZ_ERROR_INVALID_VALUE
    for mask, tagged in [(0, 1), (0x20, 1), (0x3F, 1), (0x03, 0), (0x1F, 0), (0, 0), (0x04, 2)]:
        assert lib.pz_compress_ex(fake, 100, 0, 16, mask, tagged, fake, 1000, fake, None) == bad
        assert lib.pz_compressed_size_ex(fake, 100, 0, 16, mask, tagged, fake, None, None) == bad
        assert lib.pz_decompress_ex(fake, 1000, 0, 16, mask, tagged, fake, 100, None, None) == bad



def test_rejects_bad_sampled_size_arguments_on_host(lib):
    from lossless_bit_plane_amd import _lib

    fake = 256  # aligned, never dereferenced: every call below fails its checks first
    bad = _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compressed_size_sampled(fake, 100, 0, 16, 0, fake, None, None) == bad  # stride 0
    assert lib.pz_compressed_size_sampled(fake, 100, 0, 16, 4, None, None, None) == bad  # no output
    assert lib.pz_compressed_size_sampled(fake, 100, 0, 16, 4, fake + 4, None, None) == bad  # misaligned
    assert lib.pz_compressed_size_sampled(fake, 100, 0, 16, 4, fake, fake + 1, None) == bad
    assert lib.pz_compressed_size_sampled(fake, 100, 1, 16, 4, fake, None, None) == bad  # FP32 with w=16
    assert lib.pz_compressed_size_sampled(None, 100, 0, 16, 4, fake, None, None) == bad


def test_batch_calls_check_every_tensor_before_enqueueing(lib):
    from lossless_bit_plane_amd import _lib

    fake = 256  # aligned, never dereferenced: every call below fails its checks first
    vp, sz = ctypes.c_void_p, ctypes.c_size_t

    def ptrs(*v):
        return (vp * len(v))(*v)

    def sizes(*v):
        return (sz * len(v))(*v)

    bad, short = _lib.PZ_ERROR_INVALID_VALUE, _lib.PZ_ERROR_INSUFFICIENT_BUFFER
    # An empty batch enqueues nothing and succeeds (no device needed).
    assert lib.pz_compress_batch(0, None, None, 0, 16, None, None, None, None) == 0
    assert lib.pz_decompress_batch(0, None, None, 0, 16, None, None, None, None) == 0
    assert lib.pz_compress_batch(-1, None, None, 0, 16, None, None, None, None) == bad
    assert lib.pz_compress_batch(2, None, sizes(1, 1), 0, 16, ptrs(fake, fake), sizes(9, 9), fake, None) == bad
    # The second tensor fails: misaligned source, null destination, short
    # capacity, a bad (dtype, width) pair for all.
    ok_cap = 2 + 4096
    assert lib.pz_compress_batch(2, ptrs(fake, fake + 4), sizes(4096, 4096), 0, 16, ptrs(fake, fake),
                                 sizes(ok_cap, ok_cap), fake, None) == bad
    assert lib.pz_compress_batch(2, ptrs(fake, fake), sizes(4096, 4096), 0, 16, ptrs(fake, None),
                                 sizes(ok_cap, ok_cap), fake, None) == bad
    assert lib.pz_compress_batch(2, ptrs(fake, fake), sizes(4096, 4097), 0, 16, ptrs(fake, fake),
                                 sizes(ok_cap, ok_cap), fake, None) == short
    assert lib.pz_compress_batch(2, ptrs(fake, fake), sizes(4096, 4096), 1, 16, ptrs(fake, fake),
                                 sizes(ok_cap, ok_cap), fake, None) == bad
    assert lib.pz_compress_batch(1, ptrs(fake), sizes(4096), 0, 16, ptrs(fake), sizes(ok_cap), fake + 4,
                                 None) == bad  # misaligned sizes array
    # Decompress: a stream shorter than its header table, a misaligned status.
    assert lib.pz_decompress_batch(2, ptrs(fake, fake), sizes(100, 3), 0, 16, ptrs(fake, fake),
                                   sizes(4096, 8193), None, None) == _lib.PZ_ERROR_CORRUPT_STREAM
    assert lib.pz_decompress_batch(1, ptrs(fake), sizes(100), 0, 16, ptrs(fake), sizes(4096), fake + 2,
                                   None) == bad
    assert lib.pz_decompress_batch(2, ptrs(fake, None), sizes(100, 100), 0, 16, ptrs(fake, fake),
                                   sizes(4096, 4096), None, None) == bad
    # Size batches: empty, bad pair, misaligned source or outputs.
    assert lib.pz_compressed_size_batch(0, None, None, 0, 16, None, None, None) == 0
    assert lib.pz_compressed_size_batch(1, ptrs(fake), sizes(100), 1, 16, fake, None, None) == bad
    assert lib.pz_compressed_size_batch(2, ptrs(fake, fake + 8), sizes(100, 100), 0, 16, fake, None, None) == bad
    assert lib.pz_compressed_size_batch(1, ptrs(fake), sizes(100), 0, 16, fake + 4, None, None) == bad
    assert lib.pz_compressed_size_batch(1, ptrs(fake), sizes(100), 0, 16, fake, ptrs(fake + 1), None) == bad
    assert lib.pz_compressed_size_batch(1, ptrs(None), sizes(100), 0, 16, fake, None, None) == bad


def test_swapper_rejects_bad_sizes_without_touching_the_device(lib):
    # Argument checks come before any allocation; without a GPU every valid
    # request fails too (NULL, no crash).
    for args in [(0, 4, 1 << 20, 2), (1000, 4, 1 << 20, 2), (1 << 16, 0, 1 << 20, 2),
                 (1 << 16, 4, 0, 2), (1 << 16, 4, 1 << 20, 0), (1 << 16, 4, 1 << 20, 65)]:
        assert not lib.pz_swapper_create(*args)
    assert lib.pz_swapper_free_chunks(None) == 0
    lib.pz_swapper_destroy(None)
    from lossless_bit_plane_amd import _lib

    assert lib.pz_swap_wait(None, 1, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_swap_release(None, 1) == _lib.PZ_ERROR_INVALID_VALUE


def test_noalloc_compress_rejects_on_host(lib):
    """The allocation-free compress call checks its arguments and its size
    limit before it touches the device (none of these pointers is read)."""
    from lossless_bit_plane_amd import _lib

    fake = 256
    big = _lib.PZ_NOALLOC_MAX_BYTES + 1
    cap = 2 * ((big + 4095) // 4096) + big
    assert lib.pz_compress_noalloc(fake, big, 0, 16, fake, cap, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress_noalloc(fake, 100, 0, 8, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress_noalloc(None, 100, 0, 16, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress_noalloc(fake, 100, 0, 16, fake, 1000, None, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress_noalloc(fake, 100, 0, 16, fake, 1000, fake + 4, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress_noalloc(fake + 4, 100, 0, 16, fake, 1000, fake, None) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress_noalloc(fake, 4097, 0, 16, fake, 4100, fake, None) == _lib.PZ_ERROR_INSUFFICIENT_BUFFER


def test_stream_per_thread_is_refused_on_host(lib):
    """The scratch cache is keyed by the stream handle, which hipStreamPerThread
    does not identify: compress and decompress refuse it before touching the
    device (hipStreamPerThread is the handle value 2)."""
    from lossless_bit_plane_amd import _lib

    fake, per_thread = 256, 2
    assert lib.pz_compress(fake, 100, 0, 16, fake, 1000, fake, per_thread) == _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_decompress(fake, 1000, 0, 16, fake, 100, None, per_thread) == _lib.PZ_ERROR_INVALID_VALUE
    srcs = (ctypes.c_void_p * 1)(fake)
    sizes = (ctypes.c_size_t * 1)(100)
    caps = (ctypes.c_size_t * 1)(1000)
    assert lib.pz_compress_batch(1, srcs, sizes, 0, 16, srcs, caps, fake, per_thread) == _lib.PZ_ERROR_INVALID_VALUE


def test_tensors_above_the_size_ceiling_are_refused_on_host(lib):
    """Raw sizes above PZ_MAX_RAW_BYTES (the 40-bit range of the device-wide
    offset sums, with room for the header table) are refused by every call
    before it touches the device."""
    from lossless_bit_plane_amd import _lib

    fake = 256
    big = _lib.PZ_MAX_RAW_BYTES + 4096
    cap = 2 * ((big + 4095) // 4096) + big
    inv = _lib.PZ_ERROR_INVALID_VALUE
    assert lib.pz_compress(fake, big, 0, 16, fake, cap, fake, None) == inv
    assert lib.pz_decompress(fake, cap, 0, 16, fake, big, None, None) == inv
    assert lib.pz_compressed_size(fake, big, 0, 16, fake, None, None) == inv
    assert lib.pz_compressed_size_sampled(fake, big, 0, 16, 4, fake, None, None) == inv
    assert lib.pz_block_sizes(fake, big, 0, 16, fake, None, None) == inv
    srcs = (ctypes.c_void_p * 2)(fake, fake)
    sizes = (ctypes.c_size_t * 2)(100, big)
    caps = (ctypes.c_size_t * 2)(1000, cap)
    assert lib.pz_compress_batch(2, srcs, sizes, 0, 16, srcs, caps, fake, None) == inv
    assert lib.pz_decompress_batch(2, srcs, caps, 0, 16, srcs, sizes, None, None) == inv
    assert lib.pz_compressed_size_batch(2, srcs, sizes, 0, 16, fake, None, None) == inv
