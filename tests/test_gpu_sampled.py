"""Parity of the sampled size measurement (pz_compressed_size_sampled) with
the oracle, through the C ABI (needs a GPU). The paper sizes large tensors on
every fourth 4 KB chunk (§IV "Tensor capture"); the runtime's profiling
iteration measures sizes without keeping a stream (§III-B). Bar: the sampled
chunks' header values, stream bytes and raw bytes are the oracle's exactly."""
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

    a = np.ascontiguousarray(data)
    return torch.from_numpy(a if a.size else np.zeros(16, np.uint8)).to("cuda")[: a.size]


def _check(pz, t, stride, src=None):
    print(f"[sampled] {t.name} bytes={t.nbytes} w={t.elem_bits} stride={stride}", flush=True)
    src = _dev(t.data) if src is None else src
    out, lens = pz.pz_compressed_size_sampled(src, stride, t.dtype, t.elem_bits, chunk_lens=True)
    comp, raw = (int(v) for v in out.cpu().numpy())
    o_comp, o_raw, o_H = oracle.sampled_size(t.data, t.elem_bits, stride, threads=THREADS)
    assert (comp, raw) == (o_comp, o_raw), (t.name, stride, comp, raw, o_comp, o_raw)
    np.testing.assert_array_equal(lens.cpu().numpy().view(np.uint16).astype(np.int64), o_H)
    return comp, raw


def _chunk_mix(n_chunks, tail, seed=3):
    """Chunks alternating between all-zero, random-bit and ReLU(N(0,1)) BF16
    content, so that sampled and skipped chunks differ in size."""
    rng = np.random.default_rng(seed)
    parts = []
    for c in range(n_chunks + (1 if tail else 0)):
        nb = 4096 if c < n_chunks else tail
        kind = c % 3
        if kind == 0:
            parts.append(np.zeros(nb, np.uint8))
        elif kind == 1:
            parts.append(rng.integers(0, 256, nb, dtype=np.uint8))
        else:
            x = np.maximum(rng.standard_normal((nb + 1) // 2).astype(np.float32), 0)
            parts.append(pzinputs.bf16_rne(x).view(np.uint8)[:nb])
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)


@pytest.mark.parametrize("stride", [1, 2, 3, 4, 7, 64, 1000])
def test_sampled_size_small_tensors(pz, stride):
    ts = [pzinputs.Tensor(f"mix{n}_{tail}", _chunk_mix(n, tail), 0, 16)
          for n, tail in [(1, 0), (2, 0), (13, 0), (13, 1), (13, 1000), (14, 4095), (40, 130), (0, 77)]]
    (c1,) = pzinputs.relu_smoke()
    fp32 = pzinputs.cnn_feature_maps_fp32()[0]
    ts += [c1, pzinputs.Tensor("bf16_as_w32", c1.data, 0, 32),
           pzinputs.Tensor("fp32_slice", fp32.data[: (1 << 20) + 4100].copy(), 1, 32)]
    ts += [t for t in pzinputs.edge_tensors() if t.nbytes <= (1 << 16)]
    for t in ts:
        _check(pz, t, stride)


def test_sampled_size_stride1_is_exact_size(pz):
    (t,) = pzinputs.relu_smoke()
    src = _dev(t.data)
    comp, raw = _check(pz, t, 1, src)
    size, _ = pz.pz_compressed_size(src, t.dtype, t.elem_bits)
    assert comp == int(size.item()) and raw == t.nbytes


def test_sampled_size_empty(pz):
    import torch

    src = torch.zeros(16, dtype=torch.uint8, device="cuda")[:0]
    out, lens = pz.pz_compressed_size_sampled(src, 4, 0, 16, chunk_lens=True)
    assert out.cpu().tolist() == [0, 0] and lens.numel() == 0


@pytest.mark.parametrize("name", ["cnn-fp32", "gpt2-small", "vit-layernorm", "gpt2-xl"])
def test_sampled_size_full_workloads(pz, workload_tensors, name):
    for t in workload_tensors(name):
        src = _dev(t.data)
        comp, raw = _check(pz, t, 4, src)
        size, _ = pz.pz_compressed_size(src, t.dtype, t.elem_bits)
        exact = int(size.item())
        est = t.nbytes * comp / raw
        print(f"[sampled] {t.name}: exact {exact} B, every-4th-chunk estimate {est:.0f} B "
              f"({100 * (est - exact) / exact:+.3f}%)", flush=True)
