"""pz_compress_noalloc (the compress call that allocates nothing) against
pz_compress through the C ABI: two calls in a row on one GPU, the second on
a smaller tensor, each stream and size bit-exact with pz_compress's and
nothing written past the stream."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _inputs():
    import pzinputs

    gelu, softmax, _ = pzinputs.gpt2xl_activations()
    # A tensor of several 64 KB tiles with a ragged tail, then a smaller one
    # that mixes zero and non-zero blocks, also ragged.
    first = np.concatenate([gelu.data[: 5 << 20], softmax.data[: 3 << 20], gelu.data[100: 100 + 12347]])
    second = np.ascontiguousarray(softmax.data[(64 << 20): (64 << 20) + 777_777])
    return [first, second]


def test_noalloc_matches_pz_compress_on_two_calls():
    import lossless_bit_plane_amd as pz

    dev = torch.device("cuda:0")
    for data in _inputs():
        print(f"[test_zz_no_alloc] {data.size} bytes", flush=True)
        assert data.size <= pz._lib.PZ_NOALLOC_MAX_BYTES
        src = torch.from_numpy(data).to(dev)
        ref, ref_n = pz.pz_compress(src, pz.BF16, 16)
        cap = pz.max_compressed_bytes(data.size)
        dst = torch.full((cap,), 0xA5, dtype=torch.uint8, device=dev)
        out = torch.full((1,), -1, dtype=torch.int64, device=dev)
        pz.pz_compress_noalloc(src, dst, out, pz.BF16, 16)
        torch.cuda.synchronize()
        n = int(ref_n.item())
        assert int(out.item()) == n
        assert torch.equal(dst[:n], ref[:n])
        assert bool((dst[n:] == 0xA5).all()), "bytes past the stream were written"
        back, status = pz.pz_decompress(dst, n, data.size, pz.BF16, 16)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(back[: data.size], src)
