"""Parity of the HIP codec with the CPU oracle, through the C ABI (needs a GPU).

The bar is bit-exactness: integer work, no tolerance. Checked on every
synthetic workload tensor at full size (stream bytes, header values, per-block
candidate sizes and tags, round trip), on ragged and degenerate tensors, and
on corrupt streams (status agreement with the oracle).
"""
import os

import numpy as np
import pytest

import oracle
import pzinputs
from oracle import size_model

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

    return torch.from_numpy(np.ascontiguousarray(data)).to("cuda")


def _host(t):
    return t.cpu().numpy()


def _gpu_compress(pz, t):
    src = _dev(t.data)
    dst, nbytes = pz.pz_compress(src, t.dtype, t.elem_bits)
    n = int(nbytes.item())
    return _host(dst[:n]), src


def _gpu_decompress(pz, stream_np, t):
    s = _dev(stream_np) if stream_np.size else _dev(np.zeros(16, np.uint8))
    out, status = pz.pz_decompress(s, stream_np.size, t.nbytes, t.dtype, t.elem_bits)
    return int(status.item()), _host(out[: t.nbytes])


def _check_tensor(pz, t, full_oracle=True):
    print(f"[parity] {t.name} bytes={t.nbytes} w={t.elem_bits}", flush=True)
    g_stream, src = _gpu_compress(pz, t)
    if full_oracle:
        o_stream = oracle.compress(t.data, t.elem_bits, threads=THREADS)
        assert g_stream.size == o_stream.size, (g_stream.size, o_stream.size)
        if not np.array_equal(g_stream, o_stream):
            bad = np.flatnonzero(g_stream != o_stream)
            C = oracle.num_chunks(t.nbytes)
            gH = oracle.header_table(g_stream, t.nbytes)
            oH = oracle.header_table(o_stream, t.nbytes)
            first_chunk = int(np.flatnonzero(gH != oH)[0]) if (gH != oH).any() else None
            raise AssertionError(f"stream differs at {bad.size} bytes, first at {bad[0]} (2C={2*C}); "
                                 f"first differing header chunk {first_chunk}")
    # Exact size from the size pass, and the header values.
    nbytes, lens = pz.pz_compressed_size(src, t.dtype, t.elem_bits, chunk_lens=True)
    assert int(nbytes.item()) == g_stream.size
    H = oracle.header_table(g_stream, t.nbytes)
    if lens is not None:
        np.testing.assert_array_equal(_host(lens).view(np.uint16).astype(np.int64), H)
    # Round trip of the GPU stream on the GPU.
    st, back = _gpu_decompress(pz, g_stream, t)
    assert st == 0
    assert np.array_equal(back, t.data)
    return g_stream


def test_library_symbols(pz):
    from lossless_bit_plane_amd import _lib

    for name in _lib.EXPORTS:
        assert getattr(_lib.lib, name)


def test_block_sizes_match_oracle_relu_smoke(pz):
    (t,) = pzinputs.relu_smoke()
    sizes, tags = pz.pz_block_sizes(_dev(t.data), t.dtype, t.elem_bits)
    g = _host(sizes).view(np.uint16).astype(np.int64)
    model = size_model.candidate_sizes(t.data.reshape(-1, 128), 16)
    np.testing.assert_array_equal(g, model)
    np.testing.assert_array_equal(_host(tags), size_model.select(model))


@pytest.mark.parametrize("w", [16, 32])
def test_block_sizes_match_oracle_structured(pz, w):
    """Per-candidate sizes on structured blocks: every non-zero count, single
    non-zero symbols, constants, the corner blocks."""
    rng = np.random.default_rng(w)
    N = 1024 // w
    dt = "<u2" if w == 16 else "<u4"
    rows = []
    for n in range(N + 1):
        for kind in range(6):
            s = np.zeros(N, dtype=np.uint64)
            pos = rng.choice(N, size=n, replace=False)
            if kind == 0:
                vals = rng.integers(1, 1 << w, n, dtype=np.uint64)
            elif kind == 1:
                vals = (0x3E00 if w == 16 else 0x3E000000) | rng.integers(1, 1 << (w // 2), n, dtype=np.uint64)
            elif kind == 2:
                vals = np.ones(n, np.uint64) << rng.integers(0, w, n).astype(np.uint64)
            elif kind == 3:
                vals = np.full(n, (1 << w) - 1, dtype=np.uint64)
            elif kind == 4:
                vals = np.full(n, 0x3F80 if w == 16 else 0x3F800000, dtype=np.uint64)
            else:
                vals = np.sort(rng.integers(1, 1 << 12, n, dtype=np.uint64))
            s[pos] = vals
            rows.append(s.astype(dt))
    for v in [0, 1, 0x8000, 0x7F80, 0xFFFF, 0x3F80, 0x1234]:
        rows.append(np.full(N, v, dtype=dt))
    blocks = np.stack(rows).view(np.uint8).reshape(-1)
    if w == 16:
        blocks = np.concatenate([blocks, pzinputs.corner_blocks().view(np.uint8).reshape(-1)])
    t = pzinputs.Tensor(f"structured_w{w}", blocks, 0 if w == 16 else 1, w)
    sizes, tags = pz.pz_block_sizes(_dev(t.data), t.dtype, w)
    g = _host(sizes).view(np.uint16).astype(np.int64)
    model = size_model.candidate_sizes(blocks.reshape(-1, 128), w)
    bad = np.argwhere(g != model)
    assert bad.size == 0, f"first mismatches (block, cand): {bad[:8].tolist()} gpu={g[bad[0][0]].tolist()} oracle={model[bad[0][0]].tolist()}"
    np.testing.assert_array_equal(_host(tags), size_model.select(model))
    _check_tensor(pz, t)


def test_pz_debug_dump_matches_oracle_tags(pz, monkeypatch, capfd):
    """PZ_DEBUG=1 prints the size pass's tag histogram; it equals the
    oracle's size model on the smoke tensor."""
    (t,) = pzinputs.relu_smoke()
    monkeypatch.setenv("PZ_DEBUG", "1")
    pz.pz_compressed_size(_dev(t.data), t.dtype, t.elem_bits)
    err = capfd.readouterr().err
    line = [l for l in err.splitlines() if l.startswith("[PZ_DEBUG]")][0]
    model = size_model.candidate_sizes(t.data.reshape(-1, 128), 16)
    want = np.bincount(size_model.select(model), minlength=5)
    names = ("ZVC", "DBX", "BX", "ZBX", "RAW")
    assert "tags " + ", ".join(f"{n} {c}" for n, c in zip(names, want.tolist())) in line, line
    assert f"{t.nbytes // 128} blocks" in line


def test_relu_smoke_stream_bitexact(pz):
    (t,) = pzinputs.relu_smoke()
    _check_tensor(pz, t)


@pytest.mark.parametrize("name", ["cnn-fp32", "gpt2-small", "vit-layernorm", "gpt2-xl"])
def test_workload_streams_bitexact(pz, workload_tensors, name):
    for t in workload_tensors(name):
        _check_tensor(pz, t)


def test_edge_tensors(pz):
    for t in pzinputs.edge_tensors():
        _check_tensor(pz, t)


def test_dropout_mask_and_indices(pz):
    for t in (pzinputs.dropout_mask(1 << 20), pzinputs.int64_indices(1 << 17)):
        _check_tensor(pz, t)


def test_empty_tensor(pz):
    import torch

    src = torch.zeros(16, dtype=torch.uint8, device="cuda")[:0]
    dst, nbytes = pz.pz_compress(src, 0, 16)
    assert int(nbytes.item()) == 0
    out, status = pz.pz_decompress(torch.zeros(16, dtype=torch.uint8, device="cuda"), 0, 0, 0, 16)
    assert int(status.item()) == 0
    out, status = pz.pz_decompress(torch.zeros(16, dtype=torch.uint8, device="cuda"), 4, 0, 0, 16)
    assert int(status.item()) == 3


def test_deterministic_streams(pz, workload_tensors):
    """Repeated runs give byte-identical streams (catches look-back and LDS
    races)."""
    t = workload_tensors("gpt2-small")[1]
    src = _dev(t.data)
    first = None
    for _ in range(5):
        dst, nbytes = pz.pz_compress(src, t.dtype, t.elem_bits)
        cur = _host(dst[: int(nbytes.item())])
        if first is None:
            first = cur
        else:
            assert np.array_equal(cur, first)


def test_oracle_streams_decode_on_gpu(pz, workload_tensors):
    """The GPU decoder reads the oracle's streams (the same bytes if parity
    holds, decoded independently here)."""
    for t in workload_tensors("cnn-fp32") + workload_tensors("vit-layernorm"):
        o_stream = oracle.compress(t.data, t.elem_bits, threads=THREADS)
        st, back = _gpu_decompress(pz, o_stream, t)
        assert st == 0 and np.array_equal(back, t.data)


@pytest.mark.parametrize("w", [16, 32])
def test_corrupt_streams_status_matches_oracle(pz, w):
    """Random bit flips, truncations and header edits: the GPU status equals
    the oracle's, and a good stream decodes. 16-bit symbols (ReLU BF16) and
    32-bit symbols (ReLU FP32, whose walk takes 8 lanes per chunk)."""
    if w == 16:
        (base,) = pzinputs.relu_smoke()
        data = base.data[: 24 * 4096 + 777].copy()
    else:
        x = np.random.default_rng(23).standard_normal(24 * 1024 + 200, dtype=np.float32)
        data = np.maximum(np.float32(0.5) * x, np.float32(0)).view(np.uint8)[: 24 * 4096 + 777].copy()
    t = pzinputs.Tensor("corrupt_base", data, 0 if w == 16 else 1, w)
    stream = oracle.compress(data, w)
    rng = np.random.default_rng(9)
    C = oracle.num_chunks(data.size)
    cases = []
    for _ in range(60):
        s = stream.copy()
        pos = int(rng.integers(2 * C, s.size))
        s[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        cases.append(s)
    for _ in range(10):
        s = stream.copy()
        c = int(rng.integers(0, C))
        h = int(s[2 * c]) | (int(s[2 * c + 1]) << 8)
        h2 = max(0, h + int(rng.integers(-3, 4)))
        s[2 * c], s[2 * c + 1] = h2 & 0xFF, h2 >> 8
        cases.append(s)
    cases.append(stream[:-1].copy())
    cases.append(np.concatenate([stream, np.zeros(3, np.uint8)]))
    agree = 0
    for s in cases:
        o = oracle.decompress_status(s, data.size, w)
        st, back = _gpu_decompress(pz, s, t)
        assert st == (0 if o == oracle.OK else 3), (o, st)
        if o == oracle.OK:
            assert np.array_equal(back, oracle.decompress(s, data.size, w))
        agree += 1
    assert agree == len(cases)


def test_scratch_reuse_across_calls(pz):
    """Back-to-back calls on one stream reuse its scratch (epoch-tagged
    look-back words, a tile counter that keeps counting): sizes that grow and
    shrink, a corrupt stream between good ones (its status must not leak into
    the next call), and a second stream interleaved with the first."""
    import torch

    (base,) = pzinputs.relu_smoke()
    sizes = [base.nbytes, 4096 * 3 + 5, 700_000, 77, base.nbytes - 4096, 4096 * 70, 1]
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    for k, n in enumerate(sizes):
        data = base.data[-n:].copy() if k % 2 else base.data[:n].copy()
        t = pzinputs.Tensor(f"reuse_{k}", data, 0, 16)
        s = streams[k % 2]
        with torch.cuda.stream(s):
            src = _dev(data)
            dst, nbytes = pz.pz_compress(src, 0, 16, stream=s)
            s.synchronize()
            g = _host(dst[: int(nbytes.item())])
            assert np.array_equal(g, oracle.compress(data, 16)), t.name
            if k == 3:
                bad = g.copy()
                bad[-1] ^= 0x80  # padding bit or payload bit: either way corrupt or a different decode
                o = oracle.decompress_status(bad, n, 16)
                out, status = pz.pz_decompress(_dev(bad), bad.size, n, 0, 16, stream=s)
                s.synchronize()
                assert int(status.item()) == (0 if o == oracle.OK else 3)
            out, status = pz.pz_decompress(_dev(g), g.size, n, 0, 16, stream=s)
            s.synchronize()
            assert int(status.item()) == 0, t.name
            assert np.array_equal(_host(out[:n]), data), t.name
