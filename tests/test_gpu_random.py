"""Randomized parity with the oracle (needs a GPU): seeded tensors of random
length whose chunks mix the structures the codec distinguishes (all-zero,
sparse, random bits, smooth values, constant runs, sign alternation), every
allowed (dtype, symbol width) pair, the plain calls, random codec variants
and batched calls on random sets of such tensors. Bar: stream, size pass and
sampled size bit-exact with the oracle; the round trip restores the
bytes."""
import os

import numpy as np
import pytest

import oracle
import pzinputs

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
PAIRS = [(0, 16), (0, 32), (1, 32), (2, 32)]  # (dtype, elem_bits)
MODES = [(0x1F, True), (0x1F, True), (0x1F, True), (0x01, False), (0x02, False), (0x04, False),
         (0x08, False), (0x10, False), (0x0B, True), (0x16, True)]


@pytest.fixture(scope="module")
def pz():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bit_plane_amd as pz

    return pz


def _chunk(rng, nbytes):
    kind = rng.integers(0, 7)
    if kind == 0:
        return np.zeros(nbytes, np.uint8)
    if kind == 1:
        return rng.integers(0, 256, nbytes, dtype=np.uint8)
    if kind in (2, 3):  # sparse or dense BF16-like values
        x = rng.standard_normal((nbytes + 3) // 4).astype(np.float32)
        if kind == 2:
            x = np.maximum(x, 0) * (rng.random(x.size) < 0.3)
        b = pzinputs.bf16_rne(x) if rng.random() < 0.5 else x
        return np.ascontiguousarray(b).view(np.uint8)[:nbytes]
    if kind == 4:  # smooth ramp
        x = np.cumsum(rng.standard_normal((nbytes + 3) // 4) * 0.01).astype(np.float32)
        return x.view(np.uint8)[:nbytes]
    if kind == 5:  # constant runs
        v = rng.integers(0, 1 << 32, 4, dtype=np.uint64).astype(np.uint32)
        x = np.repeat(v, (nbytes + 15) // 16)
        return x.view(np.uint8)[:nbytes]
    x = rng.standard_normal((nbytes + 1) // 2).astype(np.float32)  # alternating signs
    x[1::2] *= -1
    return pzinputs.bf16_rne(np.abs(x) * np.where(np.arange(x.size) % 2, -1, 1)).view(np.uint8)[:nbytes]


def _tensor(rng):
    n = int(rng.choice([rng.integers(1, 5000), rng.integers(4096, 1 << 18), rng.integers(1 << 18, 3 << 20)]))
    parts, left = [], n
    while left > 0:
        k = min(left, int(rng.integers(1, 5)) * 4096 - int(rng.integers(0, 2)) * int(rng.integers(0, 4096)))
        k = max(1, k)
        parts.append(_chunk(rng, k))
        left -= k
    return np.concatenate(parts)[:n]


@pytest.mark.parametrize("seed", list(range(8)))
def test_random_tensors_bitexact(pz, seed):
    import torch

    rng = np.random.default_rng(1000 + seed)
    for case in range(6):
        data = _tensor(rng)
        dtype, bits = PAIRS[int(rng.integers(0, len(PAIRS)))]
        mask, tagged = MODES[int(rng.integers(0, len(MODES)))]
        print(f"[random] seed={seed} case={case} bytes={data.size} dtype={dtype} w={bits} "
              f"mask={mask:#x} tagged={tagged}", flush=True)
        src = torch.from_numpy(data).to("cuda")
        dst, nbytes = pz.pz_compress_ex(src, mask, tagged, dtype, bits)
        n = int(nbytes.item())
        g = dst[:n].cpu().numpy()
        o = oracle.compress(data, bits, mask, tagged, threads=THREADS)
        assert g.size == o.size and np.array_equal(g, o), (seed, case)
        size, lens = pz.pz_compressed_size_ex(src, mask, tagged, dtype, bits, chunk_lens=True)
        assert int(size.item()) == n
        np.testing.assert_array_equal(lens.cpu().numpy().view(np.uint16).astype(np.int64),
                                      oracle.header_table(o, data.size))
        if (mask, tagged) == (0x1F, True):
            stride = int(rng.integers(1, 9))
            s, _ = pz.pz_compressed_size_sampled(src, stride, dtype, bits)
            o_comp, o_raw, _ = oracle.sampled_size(data, bits, stride)
            assert [int(v) for v in s.cpu().tolist()] == [o_comp, o_raw]
        out, status = pz.pz_decompress_ex(dst, n, data.size, dtype, bits, mask, tagged)
        assert int(status.item()) == 0
        assert np.array_equal(out[: data.size].cpu().numpy(), data), (seed, case)


@pytest.mark.parametrize("seed", list(range(4)))
def test_random_batches_bitexact(pz, seed):
    """Batched calls on 1-11 random tensors of one (dtype, width) pair, some
    empty: every stream bit-exact with the oracle, every round trip exact."""
    import torch

    rng = np.random.default_rng(2000 + seed)
    for case in range(3):
        count = int(rng.integers(1, 12))
        datas = [_tensor(rng) if rng.random() < 0.85 else np.zeros(0, np.uint8) for _ in range(count)]
        dtype, bits = PAIRS[int(rng.integers(0, len(PAIRS)))]
        print(f"[random batch] seed={seed} case={case} sizes={[d.size for d in datas]} dtype={dtype} w={bits}",
              flush=True)
        srcs = [torch.from_numpy(d).to("cuda") if d.size else torch.zeros(16, dtype=torch.uint8, device="cuda")[:0]
                for d in datas]
        dsts, nb = pz.pz_compress_batch(srcs, dtype, bits)
        n = [int(v) for v in nb.cpu().tolist()]
        for i, d in enumerate(datas):
            o = oracle.compress(d, bits, threads=THREADS)
            g = dsts[i][: n[i]].cpu().numpy()
            assert g.size == o.size and np.array_equal(g, o), (seed, case, i)
        outs, status = pz.pz_decompress_batch(dsts, n, [d.size for d in datas], dtype, bits)
        assert status.cpu().tolist() == [0] * count
        for i, d in enumerate(datas):
            assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), (seed, case, i)


def _big_tensor(rng, n):
    """A tensor of n bytes from the same structures in pieces of 64 KB to
    1 MB (each piece's length a random number of whole chunks, ragged at the
    end)."""
    parts, left = [], n
    while left > 0:
        k = min(left, int(rng.integers(16, 257)) * 4096)
        parts.append(_chunk(rng, k))
        left -= k
    return np.concatenate(parts)[:n]


@pytest.mark.parametrize("seed", list(range(2)))
def test_random_batches_single_launch(pz, seed):
    """Batches of over 512 locate tiles (one 130-200 MB tensor of mixed
    structures with 1-5 small random ones, some empty), which decompress in
    the single ticketed kernel: every stream bit-exact with the oracle,
    every round trip exact."""
    import torch

    rng = np.random.default_rng(3000 + seed)
    datas = [_big_tensor(rng, int(rng.integers(130 << 20, 200 << 20)))]
    datas += [_tensor(rng) if rng.random() < 0.85 else np.zeros(0, np.uint8) for _ in range(int(rng.integers(1, 6)))]
    order = rng.permutation(len(datas))
    datas = [datas[i] for i in order]
    dtype, bits = PAIRS[int(rng.integers(0, len(PAIRS)))]
    print(f"[random batch, single launch] seed={seed} sizes={[d.size for d in datas]} dtype={dtype} w={bits}",
          flush=True)
    srcs = [torch.from_numpy(d).to("cuda") if d.size else torch.zeros(16, dtype=torch.uint8, device="cuda")[:0]
            for d in datas]
    dsts, nb = pz.pz_compress_batch(srcs, dtype, bits)
    n = [int(v) for v in nb.cpu().tolist()]
    for i, d in enumerate(datas):
        o = oracle.compress(d, bits, threads=THREADS)
        g = dsts[i][: n[i]].cpu().numpy()
        assert g.size == o.size and np.array_equal(g, o), (seed, i)
    outs, status = pz.pz_decompress_batch(dsts, n, [d.size for d in datas], dtype, bits)
    assert status.cpu().tolist() == [0] * len(datas)
    for i, d in enumerate(datas):
        assert np.array_equal(outs[i][: d.size].cpu().numpy(), d), (seed, i)
