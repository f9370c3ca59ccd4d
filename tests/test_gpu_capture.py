"""HIP graph capture. The compress and decompress calls that keep their
scratch per stream refuse a capturing stream (nothing is enqueued), while
pz_compress_noalloc runs inside a captured graph: each of several replays,
with eager work and synchronizations between them, must give the eager
stream byte for byte."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _data():
    import pzinputs

    gelu, softmax, _ = pzinputs.gpt2xl_activations()
    return np.concatenate([softmax.data[: 2 << 20], gelu.data[: 1 << 20], gelu.data[7: 7 + 5555]])


def test_cached_scratch_calls_refuse_a_capturing_stream():
    import lossless_bit_plane_amd as pz
    from lossless_bit_plane_amd._lib import PZ_ERROR_INVALID_VALUE, lib

    dev = torch.device("cuda:0")
    src = torch.from_numpy(_data()).to(dev)
    n = src.numel()
    dst = torch.empty(pz.max_compressed_bytes(n), dtype=torch.uint8, device=dev)
    out = torch.empty(1, dtype=torch.int64, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    g = torch.cuda.CUDAGraph()
    results = {}
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream().cuda_stream
        results["compress"] = lib.pz_compress(src.data_ptr(), n, 0, 16, dst.data_ptr(), dst.numel(),
                                              out.data_ptr(), s)
        results["decompress"] = lib.pz_decompress(dst.data_ptr(), dst.numel(), 0, 16, src.data_ptr(), n,
                                                  status.data_ptr(), s)
    assert results == {"compress": PZ_ERROR_INVALID_VALUE, "decompress": PZ_ERROR_INVALID_VALUE}


def test_noalloc_compress_replays_in_a_graph():
    import lossless_bit_plane_amd as pz

    dev = torch.device("cuda:0")
    data = _data()
    src = torch.from_numpy(data).to(dev)
    ref, ref_n = pz.pz_compress(src, pz.BF16, 16)
    torch.cuda.synchronize()
    n = int(ref_n.item())
    dst = torch.empty(pz.max_compressed_bytes(data.size), dtype=torch.uint8, device=dev)
    out = torch.empty(1, dtype=torch.int64, device=dev)
    pz.pz_compress_noalloc(src, dst, out, pz.BF16, 16)  # outside capture first (device set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pz.pz_compress_noalloc(src, dst, out, pz.BF16, 16)
    other = torch.from_numpy(data[::-1].copy()).to(dev)
    for rep in range(3):
        # Eager work between replays, then clear the outputs with kernels.
        pz.pz_compress(other, pz.BF16, 16)
        dst.zero_()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(out.item()) == n, rep
        assert torch.equal(dst[:n], ref[:n]), rep
