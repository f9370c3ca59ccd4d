"""Batched calls through the C ABI (needs a GPU): pz_compress_batch,
pz_compressed_size_batch and pz_decompress_batch give every tensor exactly
the stream, size, header values, output and status that the oracle fixes
for it alone. Bar: bit-exact streams and round trips,
corruption reported for the corrupt tensor only, host-side rejection of a
whole call before anything is enqueued."""
import os

import numpy as np
import pytest

import oracle
import pzinputs

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def pz():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bit_plane_amd as pz

    return pz


def _dev(data):
    import torch

    d = np.ascontiguousarray(data)
    if d.size == 0:
        return torch.zeros(16, dtype=torch.uint8, device="cuda")[:0]
    return torch.from_numpy(d).to("cuda")


def _check_batch(pz, datas, dtype, w):
    """Compress `datas` in one batch call, compare every stream with the
    oracle, decompress them in one batch call and compare the bytes."""
    srcs = [_dev(d) for d in datas]
    dsts, nb = pz.pz_compress_batch(srcs, dtype, w)
    sizes, lens = pz.pz_compressed_size_batch(srcs, dtype, w, chunk_lens=True)
    n = [int(v) for v in nb.cpu().tolist()]
    assert [int(v) for v in sizes.cpu().tolist()] == n
    for i, d in enumerate(datas):
        o = oracle.compress(d, w, threads=THREADS)
        g = dsts[i][: n[i]].cpu().numpy()
        assert g.size == o.size and np.array_equal(g, o), (i, d.size, g.size, o.size)
        np.testing.assert_array_equal(lens[i].cpu().numpy().view(np.uint16).astype(np.int64),
                                      oracle.header_table(o, d.size))
    outs, status = pz.pz_decompress_batch(dsts, n, [d.size for d in datas], dtype, w)
    assert status.cpu().tolist() == [0] * len(datas)
    for i, d in enumerate(datas):
        assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), i
    return dsts, n


def test_batch_bench_workload_bitexact(pz):
    """The GPT-2-XL BF16 workload (MLP GELU 8x1024x6400, causal softmax
    8x25x1024x1024, residual 8x1024x1600) at full size in one batch per
    direction, as the bench launches it."""
    ts = pzinputs.gpt2xl_activations()
    print("[batch] gpt2-xl workload", [t.nbytes for t in ts], flush=True)
    _check_batch(pz, [t.data for t in ts], ts[0].dtype, ts[0].elem_bits)


def test_batch_fp32_tensors(pz):
    """FP32 with 32-bit symbols: CNN feature maps and the ViT LayerNorm
    output."""
    ts = [t for t in pzinputs.cnn_feature_maps_fp32() + pzinputs.vit_layernorm() if t.elem_bits == 32]
    print("[batch] fp32", [t.name for t in ts], flush=True)
    _check_batch(pz, [t.data for t in ts], pzinputs.FP32, 32)


@pytest.mark.parametrize("w", [16, 32])
def test_batch_ragged_empty_and_split(pz, w):
    """Thirteen tensors (three empty) of ragged sizes, mixing sparse, random,
    zero and smooth bytes: two launches of up to eight tensors, empty tensors
    set directly, streams ordered densest first inside a launch."""
    rng = np.random.default_rng(70 + w)
    (base,) = pzinputs.relu_smoke()
    sizes = [0, 1, 127, 128, 4095, 4096, 4097, 65836, 0, 12345, 3 * 4096, 200000, 0, 5]
    datas = []
    for k, n in enumerate(sizes):
        if k % 4 == 0:
            d = base.data[1000 * k: 1000 * k + n]
        elif k % 4 == 1:
            d = rng.integers(0, 256, n, dtype=np.uint8)
        elif k % 4 == 2:
            d = np.zeros(n, np.uint8)
        else:
            x = np.cumsum(rng.standard_normal((n + 3) // 4) * 0.01).astype(np.float32)
            d = x.view(np.uint8)[:n]
        datas.append(np.ascontiguousarray(d))
    print(f"[batch] ragged w={w}", [d.size for d in datas], flush=True)
    dsts, n = _check_batch(pz, datas, pzinputs.BF16, w)
    assert [n[i] for i, d in enumerate(datas) if d.size == 0] == [0, 0, 0]


def test_batch_single_launch_ragged_bf16(pz):
    """One decompress launch of the single kernel (over 512 locate tiles):
    the GPT-2 attention probabilities (201 MB, 768 tiles) with seven small
    ragged tensors whose last locate tiles hold 1 to 63 chunks, so that the
    decode groups past each tensor's end are skipped (a decode ticket takes
    two groups: tensors of 1, 8, 49 and 65 chunks leave a ticket's second
    group past the end, and the 65-chunk tensor's second tile has three
    tickets with no group at all). Streams equal the oracle's and outputs
    equal the inputs."""
    big = pzinputs.gpt2_small_activations()[1]
    (base,) = pzinputs.relu_smoke()
    sizes = [1, 8 * 4096 - 1, 8 * 4096 + 1, 64 * 4096 + 2, 65 * 4096 - 2, 7 * 4096 + 100, 200000]
    datas = [big.data] + [np.ascontiguousarray(base.data[(3001 * i) % 8192:][:n]) for i, n in enumerate(sizes)]
    print("[batch] single-launch decompress, ragged BF16", [d.size for d in datas], flush=True)
    _check_batch(pz, datas, pzinputs.BF16, 16)


def test_batch_tile_edges(pz):
    """Tensors ending exactly at, one byte before and one byte after the
    tiles' edges (8 chunks per decode group, 16 per compress tile, 64 per
    locate tile), so that one tensor's last tile and the next one's first
    meet at every kind of edge in one launch."""
    (base,) = pzinputs.relu_smoke()
    sizes = []
    for chunks in (8, 16, 64, 1, 63, 65, 17, 7):
        for d in (-1, 0, 1):
            sizes.append(chunks * 4096 + d)
    datas = [np.ascontiguousarray(base.data[(977 * i) % 4096:][:n]) for i, n in enumerate(sizes)]
    print("[batch] tile edges", sizes, flush=True)
    _check_batch(pz, datas, pzinputs.BF16, 16)


def test_batch_corrupt_stream_flags_only_its_tensor(pz):
    import torch

    from lossless_bit_plane_amd._lib import PlaneZipError

    (base,) = pzinputs.relu_smoke()
    datas = [base.data[: 20 * 4096], base.data[100000: 100000 + 9 * 4096 + 55], base.data[300000: 300000 + 40000]]
    streams = [oracle.compress(d, 16) for d in datas]
    rng = np.random.default_rng(5)
    # A bit flip in the second stream that the oracle rejects.
    for _ in range(200):
        s = streams[1].copy()
        pos = int(rng.integers(2 * oracle.num_chunks(datas[1].size), s.size))
        s[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        if oracle.decompress_status(s, datas[1].size, 16) != oracle.OK:
            break
    else:
        pytest.fail("no rejected flip found")
    bad = [streams[0], s, streams[2]]
    srcs = [_dev(x) for x in bad]
    print("[batch] corrupt middle stream", flush=True)
    outs, status = pz.pz_decompress_batch(srcs, [x.size for x in bad], [d.size for d in datas], 0, 16)
    assert status.cpu().tolist() == [0, 3, 0]
    for i in (0, 2):
        assert np.array_equal(outs[i][: datas[i].size].cpu().numpy(), datas[i])
    # The next call on the same stream starts clean.
    outs, status = pz.pz_decompress_batch([_dev(x) for x in streams], [x.size for x in streams],
                                          [d.size for d in datas], 0, 16)
    assert status.cpu().tolist() == [0, 0, 0]
    # A stream shorter than its header table fails the whole call on the
    # host, and nothing is enqueued (the status words keep their sentinel).
    sentinel = torch.full((3,), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(PlaneZipError):
        pz.pz_decompress_batch([_dev(x) for x in streams], [streams[0].size, 3, streams[2].size],
                               [d.size for d in datas], 0, 16, status=sentinel)
    torch.cuda.synchronize()
    assert sentinel.cpu().tolist() == [7, 7, 7]


def _rejected_flip(stream, raw_bytes, w, chunk, rng):
    """A copy of `stream` with one payload bit of `chunk` flipped such that
    the oracle rejects that chunk decoded on its own (a one-chunk stream:
    its header, then its payload); chunks decode independently of each
    other once the headers place them."""
    H = oracle.header_table(stream, raw_bytes).astype(np.int64)
    assert H[chunk] < min(4096, raw_bytes - 4096 * chunk), "pick a coded chunk"
    off = 2 * H.size + int(H[:chunk].sum())
    raw_len = min(4096, raw_bytes - 4096 * chunk)
    for _ in range(200):
        pay = stream[off: off + H[chunk]].copy()
        i = int(rng.integers(0, pay.size))
        pay[i] ^= np.uint8(1 << int(rng.integers(0, 8)))
        one = np.concatenate([np.array([H[chunk]], dtype="<u2").view(np.uint8), pay])
        if oracle.decompress_status(one, raw_len, w) != oracle.OK:
            s = stream.copy()
            s[off + i] = pay[i]
            return s
    pytest.fail("no rejected flip found")


def test_batch_single_launch_corruption_fp32(pz):
    """Eight FP32 CNN tensors in one batch (784 locate tiles: the single
    decompress kernel, 32-bit symbols), two of them corrupt, one in a chunk
    of its last locate tile and one in a middle chunk, and one ragged at its
    end: only the corrupt tensors report corruption, every other output is
    exact; a clean batch on the same stream afterwards reports none."""
    (t,) = pzinputs.cnn_feature_maps_fp32()
    full = t.data
    ragged = full[: full.size - 5 * 4096 - 20]
    good = oracle.compress(full, 32, threads=THREADS)
    good_r = oracle.compress(ragged, 32, threads=THREADS)
    H = oracle.header_table(good, full.size)
    coded = np.flatnonzero(H < 4096)
    rng = np.random.default_rng(17)
    bad_last = _rejected_flip(good, full.size, 32, int(coded[-1]), rng)
    bad_mid = _rejected_flip(good, full.size, 32, int(coded[coded.size // 2]), rng)
    assert int(coded[-1]) >= oracle.num_chunks(full.size) - 64
    assert oracle.decompress_status(bad_last, full.size, 32) != oracle.OK
    assert oracle.decompress_status(bad_mid, full.size, 32) != oracle.OK
    streams = [good, bad_last, good_r, good, bad_mid, good, good, good]
    datas = [full, full, ragged, full, full, full, full, full]
    expect = [0, 3, 0, 0, 3, 0, 0, 0]
    print("[batch] single-launch decompress, two corrupt FP32 tensors of eight", flush=True)
    outs, status = pz.pz_decompress_batch([_dev(x) for x in streams], [x.size for x in streams],
                                          [d.size for d in datas], pzinputs.FP32, 32)
    assert status.cpu().tolist() == expect
    for i, d in enumerate(datas):
        if expect[i] == 0:
            assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), i
    clean = [good if x is not good_r else good_r for x in streams]
    outs, status = pz.pz_decompress_batch([_dev(x) for x in clean], [x.size for x in clean],
                                          [d.size for d in datas], pzinputs.FP32, 32)
    assert status.cpu().tolist() == [0] * 8
    for i, d in enumerate(datas):
        assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), i


def test_batch_single_launch_length_corruption_fp32(pz):
    """Six FP32 CNN tensors in one batch (588 locate tiles: the single
    decompress kernel): one stream with 16 trailing bytes and one a byte
    short, both corrupt for the oracle (the header sum must equal the
    stream's length), report corruption; the others decompress exactly."""
    (t,) = pzinputs.cnn_feature_maps_fp32()
    d = t.data
    good = oracle.compress(d, 32, threads=THREADS)
    long_ = np.concatenate([good, np.zeros(16, np.uint8)])
    short = good[:-1]
    assert oracle.decompress_status(long_, d.size, 32) != oracle.OK
    assert oracle.decompress_status(short, d.size, 32) != oracle.OK
    streams = [good, long_, good, short, good, good]
    print("[batch] single-launch decompress, length-corrupt FP32 streams", flush=True)
    outs, status = pz.pz_decompress_batch([_dev(x) for x in streams], [x.size for x in streams],
                                          [d.size] * len(streams), pzinputs.FP32, 32)
    assert status.cpu().tolist() == [0, 3, 0, 3, 0, 0]
    for i in (0, 2, 4, 5):
        assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), i


def test_batch_two_kernel_fp32_eight_lanes(pz):
    """Five FP32 CNN tensors in one batch: 490 tiles of 64 chunks, just
    under the single kernel's threshold, so locate walks with 8 lanes per
    chunk in 980 tiles of 32 chunks. A length-corrupt stream in the middle
    reports corruption; the others decompress exactly."""
    (t,) = pzinputs.cnn_feature_maps_fp32()
    d = t.data
    good = oracle.compress(d, 32, threads=THREADS)
    long_ = np.concatenate([good, np.zeros(16, np.uint8)])
    assert oracle.decompress_status(long_, d.size, 32) != oracle.OK
    streams = [good, good, long_, good, good]
    print("[batch] two-kernel decompress, five FP32 streams (8 lanes per chunk)", flush=True)
    outs, status = pz.pz_decompress_batch([_dev(x) for x in streams], [x.size for x in streams],
                                          [d.size] * len(streams), pzinputs.FP32, 32)
    assert status.cpu().tolist() == [0, 0, 3, 0, 0]
    for i in (0, 1, 3, 4):
        assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), i


def test_batch_single_launch_concurrent_streams(pz):
    """Two single-kernel decompress launches (768 and 588 locate tiles) on
    two streams with nothing ordering them, three times over: each stream's
    scratch (tile counter, located-tile counter, look-back words and flags)
    is its own and every wait is on a started workgroup of the same launch,
    so both round trips stay exact."""
    import torch

    big = pzinputs.gpt2_small_activations()[1]
    (cnn,) = pzinputs.cnn_feature_maps_fp32()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    jobs = [([big.data], pzinputs.BF16, 16), ([cnn.data] * 6, pzinputs.FP32, 32)]
    comp = []
    for (datas, dtype, w), s in zip(jobs, streams):
        with torch.cuda.stream(s):
            srcs = [_dev(d) for d in datas]
            dsts, nb = pz.pz_compress_batch(srcs, dtype, w)
        s.synchronize()
        comp.append((dsts, [int(v) for v in nb.cpu().tolist()]))
    for rep in range(3):
        print(f"[batch] concurrent single-launch decompress on two streams, pass {rep}", flush=True)
        results = []
        for (datas, dtype, w), (dsts, n), s in zip(jobs, comp, streams):
            with torch.cuda.stream(s):
                results.append(pz.pz_decompress_batch(dsts, n, [d.size for d in datas], dtype, w))
        torch.cuda.synchronize()
        for (datas, _, _), (outs, status) in zip(jobs, results):
            assert status.cpu().tolist() == [0] * len(datas)
            for i, d in enumerate(datas):
                assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), (rep, i)
