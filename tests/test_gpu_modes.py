"""Parity of the codec variants (candidate masks, tagged or not) with the CPU
oracle, through the C ABI (needs a GPU).

The variants are the single-codec columns the PlaneZip paper compares with
(§V-A, Fig. 3: ZVC as in cDMA, BPC's DBX on every block, BX or ZBX alone) and
PlaneZip with a subset of its candidates. Bar: the stream, its exact size and
the round trip are bit-identical to the oracle's; a corrupt stream gets the
oracle's status.
"""
import os

import numpy as np
import pytest

import oracle
import pzinputs

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
ZVC, DBX, BX, ZBX, RAW = 1, 2, 4, 8, 16
ALL = 0x1F

# (codec_mask, tagged)
MODES = [
    (ZVC, False), (DBX, False), (BX, False), (ZBX, False), (RAW, False),
    (ALL & ~ZBX, True), (ALL & ~DBX, True), (ZVC | RAW, True), (DBX | BX, True), (ZBX, True),
]


@pytest.fixture(scope="module")
def pz():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bit_plane_amd as pz

    return pz


def _dev(data):
    import torch

    a = np.ascontiguousarray(data)
    return torch.from_numpy(a if a.size else np.zeros(16, np.uint8)).to("cuda")[: a.size]


def _tensors():
    (c1,) = pzinputs.relu_smoke()
    fp32 = pzinputs.cnn_feature_maps_fp32()[0]
    ts = [
        c1,
        pzinputs.Tensor("bf16_as_w32", c1.data, 0, 32),
        pzinputs.Tensor("fp32_slice", fp32.data[: (1 << 21) + 777].copy(), 1, 32),
        pzinputs.dropout_mask(1 << 18),
    ]
    ts += [t for t in pzinputs.edge_tensors() if t.nbytes <= (1 << 16)]
    return ts


@pytest.mark.parametrize("mask,tagged", MODES)
def test_mode_streams_bitexact(pz, mask, tagged):
    for t in _tensors():
        print(f"[modes] mask={mask:#x} tagged={tagged} {t.name} bytes={t.nbytes} w={t.elem_bits}", flush=True)
        src = _dev(t.data)
        dst, nbytes = pz.pz_compress_ex(src, mask, tagged, t.dtype, t.elem_bits)
        n = int(nbytes.item())
        g = dst[:n].cpu().numpy()
        o = oracle.compress(t.data, t.elem_bits, mask, tagged, threads=THREADS)
        assert g.size == o.size, (t.name, g.size, o.size)
        assert np.array_equal(g, o), (t.name, int(np.flatnonzero(g != o)[0]))
        size, lens = pz.pz_compressed_size_ex(src, mask, tagged, t.dtype, t.elem_bits, chunk_lens=True)
        assert int(size.item()) == n
        if lens is not None:
            np.testing.assert_array_equal(lens.cpu().numpy().view(np.uint16).astype(np.int64),
                                          oracle.header_table(g, t.nbytes))
        out, status = pz.pz_decompress_ex(_dev(g), n, t.nbytes, t.dtype, t.elem_bits, mask, tagged)
        assert int(status.item()) == 0
        assert np.array_equal(out[: t.nbytes].cpu().numpy(), t.data)


@pytest.mark.parametrize("mask,tagged", [(BX, False), (DBX, False), (ZVC | RAW, True)])
def test_mode_corrupt_streams_status_matches_oracle(pz, mask, tagged):
    (base,) = pzinputs.relu_smoke()
    data = base.data[: 24 * 4096 + 777].copy()
    stream = oracle.compress(data, 16, mask, tagged)
    rng = np.random.default_rng(11)
    C = oracle.num_chunks(data.size)
    for _ in range(40):
        s = stream.copy()
        pos = int(rng.integers(2 * C, s.size))
        s[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        o = oracle.decompress_status(s, data.size, 16, mask, tagged)
        out, status = pz.pz_decompress_ex(_dev(s), s.size, data.size, 0, 16, mask, tagged)
        st = int(status.item())
        assert st == (0 if o == oracle.OK else 3), (o, st)
        if o == oracle.OK:
            assert np.array_equal(out[: data.size].cpu().numpy(),
                                  oracle.decompress(s, data.size, 16, mask, tagged))
