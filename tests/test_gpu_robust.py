"""Memory-safety and large-size checks of the HIP codec through the C ABI
(needs a GPU).

* Canary bytes around every output: compress writes nothing past the
  stream's length, and decompress nothing outside [dst, dst + raw_bytes),
  for good and corrupt streams, single and batched calls.
* Reads stay inside the inputs: two different poison patterns placed after
  raw_bytes (compress) or comp_bytes (decompress) give identical streams,
  statuses and outputs.
* A tensor above 4 GiB of mixed content whose stream also passes 4 GiB:
  64-bit chunk offsets and look-back prefix sums beyond 2^32. Sampled chunks
  are checked byte for byte against the oracle's coding of that chunk, at
  stream offsets on both sides of 2^31 and 2^32, and the whole tensor
  round-trips.
"""
import functools

import numpy as np
import pytest

import oracle
import pzinputs

pytestmark = pytest.mark.gpu

PRE = 256          # canary bytes before a window (keeps 16-byte alignment)
POST = 4096        # canary bytes after a window's end
CANARY = 0xA5
POISONS = (0x00, 0xFF)


@pytest.fixture(scope="module")
def pz():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bit_plane_amd as pz

    return pz


def _canvas(data_or_len, fill):
    """A device buffer PRE + n + POST bytes long, filled with ``fill``, whose
    window [PRE, PRE + n) holds ``data`` (or stays filled). Returns (buf, window)."""
    import torch

    n = data_or_len if isinstance(data_or_len, int) else int(data_or_len.size)
    buf = torch.full((PRE + n + POST,), fill, dtype=torch.uint8, device="cuda")
    win = buf[PRE:PRE + n]
    if not isinstance(data_or_len, int) and n:
        win.copy_(torch.from_numpy(np.ascontiguousarray(data_or_len)))
    return buf, win


def _untouched(buf, lo, hi, fill):
    """Bytes of buf outside [lo, hi) all equal fill."""
    h = buf.cpu().numpy()
    return bool((h[:lo] == fill).all() and (h[hi:] == fill).all())


CASES = ["relu_bf16_1", "relu_bf16_127", "relu_bf16_4097", "relu_bf16_99081", "relu_bf16_300001",
         "random_bf16_70001", "mixed_bf16", "relu_fp32_200003", "mask_other_9999"]


@functools.lru_cache(maxsize=None)
def _case(name):
    """(bytes, dtype, w) of a named tensor: ragged ReLU BF16, random (raw
    chunks), mixed tiles, FP32 and 'other' data, from one byte to several
    tiles."""
    if name.startswith("relu_bf16_"):
        (smoke,) = pzinputs.relu_smoke()
        return smoke.data[:int(name.rsplit("_", 1)[1])].copy(), 0, 16
    if name == "random_bf16_70001":
        return np.random.default_rng(21).integers(0, 256, 70001, dtype=np.uint8), 0, 16
    if name == "mixed_bf16":
        return pzinputs.mixed_large(40 * 32768 + 333).data, 0, 16
    if name == "relu_fp32_200003":
        x = np.maximum(np.random.default_rng(22).standard_normal(50001, dtype=np.float32), np.float32(0))
        return x.view(np.uint8)[:200003].copy(), 1, 32
    if name == "mask_other_9999":
        return pzinputs.dropout_mask(9999).data, 2, 32
    raise KeyError(name)


def _corruptions(stream, raw_bytes, w, rng, count=6):
    """Corrupt variants of a good stream: payload bit flips the oracle rejects
    (or accepts with a different decode), a header edit, a truncation."""
    C = oracle.num_chunks(raw_bytes)
    out = []
    if stream.size > 2 * C:
        for _ in range(count):
            s = stream.copy()
            pos = int(rng.integers(2 * C, s.size))
            s[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
            out.append(s)
        out.append(stream[:-1].copy())
    s = stream.copy()
    c = int(rng.integers(0, C))
    h = int(s[2 * c]) | (int(s[2 * c + 1]) << 8)
    h2 = max(0, h - 1)
    s[2 * c], s[2 * c + 1] = h2 & 0xFF, h2 >> 8
    out.append(s)
    return out


def _compress_canaried(pz, data, dtype, w, poison):
    """Compress data placed in a poisoned source canvas into a canaried
    destination canvas; returns the stream (host) after checking the canaries."""
    import torch

    n = int(data.size)
    _, src = _canvas(data, poison)
    cap = oracle.max_compressed(n)
    dbuf, dst = _canvas(cap, CANARY)
    out_bytes = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    pz.pz_compress(src, dtype, w, dst=dst, out_bytes=out_bytes)
    m = int(out_bytes.item())
    assert 0 <= m <= cap
    assert _untouched(dbuf, PRE, PRE + m, CANARY), "compress wrote outside its stream"
    return dst[:m].cpu().numpy()


def _decompress_canaried(pz, stream, raw_bytes, dtype, w, poison):
    """Decompress a stream placed in a poisoned source canvas into a canaried
    destination canvas; returns (status, output window) after the canaries."""
    import torch

    _, src = _canvas(stream, poison)
    dbuf, dst = _canvas(raw_bytes, CANARY)
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pz.pz_decompress(src, int(stream.size), raw_bytes, dtype, w, dst=dst, status=status)
    st = int(status.item())
    assert _untouched(dbuf, PRE, PRE + raw_bytes, CANARY), "decompress wrote outside its output"
    return st, dst.cpu().numpy()


@pytest.mark.parametrize("name", CASES)
def test_canaries_and_poison_single_calls(pz, name):
    data, dtype, w = _case(name)
    n = int(data.size)
    expect = oracle.compress(data, w)
    streams = []
    for p in POISONS:
        print(f"[robust] compress {name} n={n} w={w} poison={p:#x}", flush=True)
        streams.append(_compress_canaried(pz, data, dtype, w, p))
    for s in streams:
        assert np.array_equal(s, expect), name
    rng = np.random.default_rng(1000 + CASES.index(name))
    for k, s in enumerate([expect] + _corruptions(expect, n, w, rng)):
        o = oracle.decompress_status(s, n, w)
        got = []
        for p in POISONS:
            print(f"[robust] decompress {name} variant={k} comp={s.size} poison={p:#x}", flush=True)
            got.append(_decompress_canaried(pz, s, n, dtype, w, p))
        (st0, out0), (st1, out1) = got
        assert st0 == st1 == (0 if o == oracle.OK else 3), (name, k, o, st0, st1)
        assert np.array_equal(out0, out1), (name, k, "output depends on bytes past comp_bytes")
        if o == oracle.OK:
            assert np.array_equal(out0, oracle.decompress(s, n, w)), (name, k)


def test_canaries_and_poison_batched_calls(pz):
    """Batched compress and decompress: every tensor's destination keeps its
    canaries, poison after each input changes nothing, and a corrupt stream in
    the middle of a batch is flagged alone."""
    import torch

    (smoke,) = pzinputs.relu_smoke()
    rng = np.random.default_rng(33)
    datas = [smoke.data[:5 * 4096 + 3].copy(), rng.integers(0, 256, 3 * 32768 + 17, dtype=np.uint8),
             smoke.data[200_000:200_000 + 9 * 32768].copy(), smoke.data[:1].copy()]
    expect = [oracle.compress(d, 16) for d in datas]
    runs = []
    for p in POISONS:
        print(f"[robust] compress_batch poison={p:#x}", flush=True)
        srcs = [_canvas(d, p)[1] for d in datas]
        canv = [_canvas(oracle.max_compressed(d.size), CANARY) for d in datas]
        out_bytes = torch.full((len(datas),), -1, dtype=torch.int64, device="cuda")
        pz.pz_compress_batch(srcs, 0, 16, dsts=[c[1] for c in canv], out_bytes=out_bytes)
        ms = out_bytes.cpu().tolist()
        for (buf, win), m, e in zip(canv, ms, expect):
            assert m == e.size
            assert _untouched(buf, PRE, PRE + m, CANARY), "batched compress wrote outside a stream"
            assert np.array_equal(win[:m].cpu().numpy(), e)
        runs.append(ms)
    assert runs[0] == runs[1]

    # A rejected bit flip in the third stream.
    for _ in range(500):
        bad = expect[2].copy()
        pos = int(rng.integers(2 * oracle.num_chunks(datas[2].size), bad.size))
        bad[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        if oracle.decompress_status(bad, datas[2].size, 16) != oracle.OK:
            break
    else:
        pytest.fail("no rejected flip found")
    streams = [expect[0], expect[1], bad, expect[3]]
    outs = []
    for p in POISONS:
        print(f"[robust] decompress_batch poison={p:#x}", flush=True)
        srcs = [_canvas(s, p)[1] for s in streams]
        canv = [_canvas(d.size, CANARY) for d in datas]
        status = torch.full((len(datas),), -7, dtype=torch.int32, device="cuda")
        pz.pz_decompress_batch(srcs, [s.size for s in streams], [d.size for d in datas], 0, 16,
                               dsts=[c[1] for c in canv], status=status)
        assert status.cpu().tolist() == [0, 0, 3, 0]
        for (buf, win), d in zip(canv, datas):
            assert _untouched(buf, PRE, PRE + d.size, CANARY), "batched decompress wrote outside an output"
        outs.append([c[1].cpu().numpy() for c in canv])
    for i, d in enumerate(datas):
        assert np.array_equal(outs[0][i], outs[1][i]), i
        if i != 2:
            assert np.array_equal(outs[0][i], d), i


LARGE_BYTES = 21 * (1 << 28) + 777   # 5.25 GiB + a ragged tail


def test_stream_above_4gib_mixed_content(pz):
    """5.25 GiB of mixed tiles (about 0.84 kept raw, so the stream is about
    4.4 GiB): chunk offsets and look-back sums pass 2^32. The header table is
    consistent with the reported length and the size pass, sampled chunks on
    both sides of byte 2^32 of the stream match the oracle's coding of that
    chunk, a batched call gives the same stream, and the tensor round-trips."""
    import torch

    t = pzinputs.mixed_large(LARGE_BYTES)
    n = t.nbytes
    C = oracle.num_chunks(n)
    print(f"[robust] large tensor n={n} chunks={C}", flush=True)
    src = torch.from_numpy(t.data).to("cuda")
    dst, out_bytes = pz.pz_compress(src, 0, 16)
    m = int(out_bytes.item())
    print(f"[robust] large stream bytes={m}", flush=True)
    assert m > (1 << 32) + (1 << 28), "the stream must pass 4 GiB for this test to mean anything"

    H = dst[:2 * C].cpu().numpy().view("<u2").astype(np.int64)
    assert 2 * C + int(H.sum()) == m
    size, _ = pz.pz_compressed_size(src, 0, 16)
    assert int(size.item()) == m
    off = 2 * C + np.cumsum(H) - H
    rng = np.random.default_rng(44)
    picks = {0, 1, C - 2, C - 1}
    for edge in (1 << 31, 1 << 32):   # the chunks holding stream bytes 2^31 and 2^32, and neighbours
        cross = int(np.searchsorted(off, edge, side="right")) - 1
        picks |= set(range(max(0, cross - 20), min(C, cross + 21)))
    picks |= set(int(c) for c in rng.integers(0, C, 60))
    picks |= set(int(c) for c in np.flatnonzero(off > (1 << 32))[:: 997][:20])
    for c in sorted(picks):
        raw = t.data[c * 4096:min(n, (c + 1) * 4096)]
        h, payload, _, _ = oracle.compress_chunk(raw, 16)
        assert h == H[c], (c, h, int(H[c]))
        got = dst[int(off[c]):int(off[c]) + int(H[c])].cpu().numpy()
        assert np.array_equal(got, payload), f"chunk {c} at stream offset {int(off[c])}"

    print("[robust] large batched compress", flush=True)
    small = torch.from_numpy(t.data[:5 * 4096 + 9].copy()).to("cuda")
    bdsts, bbytes = pz.pz_compress_batch([small, src], 0, 16)
    bm = bbytes.cpu().tolist()
    assert bm[1] == m
    assert torch.equal(bdsts[1][:m], dst[:m])
    assert np.array_equal(bdsts[0][:bm[0]].cpu().numpy(), oracle.compress(t.data[:5 * 4096 + 9], 16))
    del bdsts

    print("[robust] large decompress", flush=True)
    back, status = pz.pz_decompress(dst, m, n, 0, 16)
    assert int(status.item()) == 0
    # Compared a GiB at a time, so that a failure names the range.
    step = 1 << 30
    for a in range(0, n, step):
        assert torch.equal(back[a:a + step], src[a:a + step]), f"round trip differs in raw bytes [{a}, {a + step})"
    del back
    print("[robust] large batched decompress", flush=True)
    souts, bstatus = pz.pz_decompress_batch([dst, dst], [m, m], [n, n], 0, 16)
    assert bstatus.cpu().tolist() == [0, 0]
    assert torch.equal(souts[0][:n], src) and torch.equal(souts[1][:n], src)
