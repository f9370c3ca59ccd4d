"""ctypes binding of ``libplanezip.so`` (the C ABI in include/planezip.h).

Argument marshalling only: every step of the codec runs in the HIP kernels.
There is no CPU fallback; importing fails loudly if the library is missing.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libplanezip.so")

PZ_SUCCESS = 0
PZ_ERROR_INVALID_VALUE = 1
PZ_ERROR_INSUFFICIENT_BUFFER = 2
PZ_ERROR_CORRUPT_STREAM = 3
PZ_ERROR_HIP = 4
PZ_NOALLOC_MAX_BYTES = 1073545216
PZ_MAX_RAW_BYTES = 1 << 39

EXPORTS = ("pz_compressed_size", "pz_compress", "pz_decompress", "pz_block_sizes", "pz_status_string",
           "pz_compressed_size_ex", "pz_compress_ex", "pz_decompress_ex", "pz_compressed_size_sampled",
           "pz_predictor_create", "pz_predictor_destroy", "pz_predictor_update", "pz_predictor_predict",
           "pz_predictor_entries", "pz_predictor_clear",
           "pz_swapper_create", "pz_swapper_destroy", "pz_swapper_free_chunks", "pz_swap_out", "pz_swap_wait",
           "pz_swap_in", "pz_swap_release", "pz_swap_read", "pz_compress_batch", "pz_decompress_batch",
           "pz_compressed_size_batch", "pz_compress_noalloc", "pz_transfer_time")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python lossless_bit_plane_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.pz_compressed_size.argtypes = [vp, sz, i, i, vp, vp, vp]
    lib.pz_compress.argtypes = [vp, sz, i, i, vp, sz, vp, vp]
    lib.pz_compress_noalloc.argtypes = [vp, sz, i, i, vp, sz, vp, vp]
    lib.pz_decompress.argtypes = [vp, sz, i, i, vp, sz, vp, vp]
    lib.pz_block_sizes.argtypes = [vp, sz, i, i, vp, vp, vp]
    u32 = ctypes.c_uint32
    lib.pz_compressed_size_ex.argtypes = [vp, sz, i, i, u32, i, vp, vp, vp]
    lib.pz_compress_ex.argtypes = [vp, sz, i, i, u32, i, vp, sz, vp, vp]
    lib.pz_decompress_ex.argtypes = [vp, sz, i, i, u32, i, vp, sz, vp, vp]
    lib.pz_compressed_size_sampled.argtypes = [vp, sz, i, i, u32, vp, vp, vp]
    lib.pz_compress_batch.argtypes = [i, ctypes.POINTER(vp), ctypes.POINTER(sz), i, i, ctypes.POINTER(vp),
                                      ctypes.POINTER(sz), vp, vp]
    lib.pz_decompress_batch.argtypes = [i, ctypes.POINTER(vp), ctypes.POINTER(sz), i, i, ctypes.POINTER(vp),
                                        ctypes.POINTER(sz), vp, vp]
    lib.pz_compressed_size_batch.argtypes = [i, ctypes.POINTER(vp), ctypes.POINTER(sz), i, i, vp,
                                             ctypes.POINTER(vp), vp]
    u64 = ctypes.c_uint64
    lib.pz_predictor_create.argtypes = [sz]
    lib.pz_predictor_create.restype = vp
    lib.pz_predictor_destroy.argtypes = [vp]
    lib.pz_predictor_destroy.restype = None
    lib.pz_predictor_update.argtypes = [vp, u64, u64, u64]
    lib.pz_predictor_predict.argtypes = [vp, u64, u64, ctypes.POINTER(u64), ctypes.POINTER(i)]
    lib.pz_transfer_time.argtypes = [u64, ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.pz_transfer_time.restype = ctypes.c_double
    lib.pz_predictor_entries.argtypes = [vp]
    lib.pz_predictor_entries.restype = sz
    lib.pz_predictor_clear.argtypes = [vp]
    lib.pz_predictor_clear.restype = None
    lib.pz_swapper_create.argtypes = [sz, sz, sz, i]
    lib.pz_swapper_create.restype = vp
    lib.pz_swapper_destroy.argtypes = [vp]
    lib.pz_swapper_destroy.restype = None
    lib.pz_swapper_free_chunks.argtypes = [vp]
    lib.pz_swapper_free_chunks.restype = sz
    lib.pz_swap_out.argtypes = [vp, vp, sz, i, i, vp, ctypes.POINTER(u64)]
    lib.pz_swap_wait.argtypes = [vp, u64, ctypes.POINTER(u64)]
    lib.pz_swap_in.argtypes = [vp, u64, vp, vp, vp]
    lib.pz_swap_release.argtypes = [vp, u64]
    lib.pz_swap_read.argtypes = [vp, u64, vp, sz, ctypes.POINTER(u64)]
    for name in ("pz_swap_out", "pz_swap_wait", "pz_swap_in", "pz_swap_release", "pz_swap_read"):
        getattr(lib, name).restype = ctypes.c_int
    for name in ("pz_compressed_size", "pz_compress", "pz_compress_noalloc", "pz_decompress", "pz_block_sizes",
                 "pz_compressed_size_ex", "pz_compress_ex", "pz_decompress_ex", "pz_compressed_size_sampled",
                 "pz_predictor_update", "pz_predictor_predict", "pz_compress_batch", "pz_decompress_batch",
                 "pz_compressed_size_batch"):
        getattr(lib, name).restype = ctypes.c_int
    lib.pz_status_string.argtypes = [ctypes.c_int]
    lib.pz_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


class PlaneZipError(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = lib.pz_status_string(status).decode()
        super().__init__(f"{call} failed: {msg} ({status})")
        self.status = status


def check(status: int, call: str) -> None:
    if status != PZ_SUCCESS:
        raise PlaneZipError(status, call)
