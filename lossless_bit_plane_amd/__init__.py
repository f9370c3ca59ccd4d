"""PlaneZip lossless bit-plane block codec for MI355X (gfx950).

Thin Python binding of the C ABI in ``include/planezip.h``; PyTorch supplies
device memory and streams. The codec is the one of the PlaneZip paper
(§III-A, Fig. 2): every 128-byte block takes the shortest of its ZVC, DBX, BX,
ZBX and verbatim codings behind a 3-bit tag, and 4 KB chunks carry 16-bit
length headers; bit layout FORMAT.md v1.
The ``*_ex`` calls run the single-codec and reduced-candidate variants the
paper compares PlaneZip with (§V-A, Fig. 3); ``pz_compressed_size_sampled``
and the ``pz_predictor_*`` table are the runtime's size measurement and
per-tensor predictor (§III-B); ``Swapper`` and ``SwapHooks`` are the copy
path (§III, Fig. 2): compression into a pinned pool of fixed-size chunks and
back, under autograd's saved-tensor hooks.
"""
from .codec import (  # noqa: F401
    BF16, FP32, OTHER, CODEC_ALL, CODEC_BX, CODEC_DBX, CODEC_RAW, CODEC_ZBX, CODEC_ZVC,
    max_compressed_bytes, num_chunks,
    pz_block_sizes, pz_compress, pz_compressed_size, pz_decompress,
    pz_compress_ex, pz_compressed_size_ex, pz_decompress_ex, pz_compressed_size_sampled,
    pz_compress_batch, pz_decompress_batch, pz_compressed_size_batch, pz_compress_noalloc, compress, decompress,
)
from .predictor import (  # noqa: F401
    Predictor, signature, pz_predictor_create, pz_predictor_destroy, pz_predictor_update,
    pz_predictor_predict, pz_predictor_entries, pz_predictor_clear, transfer_time,
)
from .swap import Swapper, SwapHooks  # noqa: F401
