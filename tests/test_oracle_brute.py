"""Brute-force checks of the CPU oracle on tiny and structured blocks (no GPU).

Mirrors the paper's validation (§III-A "Validation": every encoder in two
implementations, the decoder reproduces every block, the bit counts agree):

* every block: all five candidates are encoded explicitly and decoded back,
  the decoder consumes exactly the encoded bits, and the bit counts equal the
  independent numpy size model;
* the chosen tag is the smallest candidate, ties to the lowest tag;
* whole streams round-trip and their length matches the size model's
  accounting of tags, headers and padding.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import size_model


def _check_blocks(blocks_u8, w, explicit=True):
    blocks = np.ascontiguousarray(blocks_u8, dtype=np.uint8).reshape(-1, 128)
    model = size_model.candidate_sizes(blocks, w)
    c_sizes = oracle.blocks_sizes(blocks, w)
    np.testing.assert_array_equal(c_sizes, model)
    if explicit:
        for b in range(blocks.shape[0]):
            for cand in range(5):
                payload, nbits = oracle.encode_candidate(blocks[b], w, cand)
                assert nbits == model[b, cand]
                back, used = oracle.decode_candidate(payload, nbits, w, cand)
                assert used == nbits
                assert back.tobytes() == blocks[b].tobytes(), (b, cand)
    stream, tags, bits = oracle.compress(blocks, w, want_blocks=True)
    np.testing.assert_array_equal(tags, size_model.select(model))
    np.testing.assert_array_equal(bits, 3 + model.min(axis=1))
    assert stream.size == size_model.stream_bytes(blocks.size, bits)
    assert oracle.decompress(stream, blocks.size, w).tobytes() == blocks.tobytes()
    return model


def test_every_constant_bf16_block():
    """All 65,536 constant BF16 blocks."""
    v = np.arange(1 << 16, dtype=np.uint64).astype("<u2")
    blocks = np.repeat(v[:, None], 64, axis=1).view(np.uint8)
    model = _check_blocks(blocks, 16, explicit=False)
    # A constant block has all-zero deltas: DBX is always the base plus one run.
    assert (model[:, 1] == 16 + 6).all()
    # Explicit encode/decode of every candidate on a spread of them.
    _check_blocks(blocks[::257], 16, explicit=True)


def test_single_nonzero_bf16_blocks():
    """One non-zero symbol: every position with 512 values, and every value
    at the first and last positions."""
    rng = np.random.default_rng(3)
    rows = []
    for pos in range(64):
        vals = rng.integers(1, 1 << 16, 512)
        b = np.zeros((vals.size, 64), dtype="<u2")
        b[:, pos] = vals
        rows.append(b)
    for pos in (0, 63):
        b = np.zeros(((1 << 16) - 1, 64), dtype="<u2")
        b[:, pos] = np.arange(1, 1 << 16)
        rows.append(b)
    blocks = np.concatenate(rows).view(np.uint8)
    _check_blocks(blocks, 16, explicit=False)
    _check_blocks(blocks[::101], 16, explicit=True)


@pytest.mark.parametrize("w", [16, 32])
def test_every_nonzero_count(w):
    """ZBX over every count n = 0..N of non-zero symbols, at random positions,
    with values sharing high bits (ReLU-like) and with random bits."""
    rng = np.random.default_rng(w)
    N = 1024 // w
    dt = "<u2" if w == 16 else "<u4"
    rows = []
    for n in range(N + 1):
        for kind in range(4):
            s = np.zeros(N, dtype=np.uint64)
            pos = rng.choice(N, size=n, replace=False)
            if kind == 0:
                vals = rng.integers(1, 1 << w, n, dtype=np.uint64)
            elif kind == 1:
                hi = (0x3E00 if w == 16 else 0x3E000000)
                vals = hi | rng.integers(1, 1 << (w // 2), n, dtype=np.uint64)
            elif kind == 2:
                vals = np.full(n, 1, dtype=np.uint64) << rng.integers(0, w, n).astype(np.uint64)
            else:
                vals = np.full(n, (1 << w) - 1, dtype=np.uint64)
            s[pos] = vals
            rows.append(s.astype(dt))
    blocks = np.stack(rows).view(np.uint8)
    _check_blocks(blocks, w, explicit=True)


SMALL_ALPHABET_16 = [0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0xFFFF]
SMALL_ALPHABET_32 = [0x0, 0x80000000, 0x3F800000, 0xBF800000, 0x7F800000, 0x7FC00000, 0x1, 0xFFFFFFFF]


@settings(max_examples=150, deadline=None)
@given(st.lists(st.sampled_from(SMALL_ALPHABET_16), min_size=64, max_size=64))
def test_small_alphabet_bf16(symbols):
    block = np.array(symbols, dtype="<u2").view(np.uint8)
    _check_blocks(block, 16, explicit=True)


@settings(max_examples=150, deadline=None)
@given(st.lists(st.sampled_from(SMALL_ALPHABET_32), min_size=32, max_size=32))
def test_small_alphabet_fp32(symbols):
    block = np.array(symbols, dtype="<u4").view(np.uint8)
    _check_blocks(block, 32, explicit=True)


@settings(max_examples=60, deadline=None)
@given(st.binary(min_size=128, max_size=128), st.sampled_from([16, 32]))
def test_arbitrary_bytes(data, w):
    _check_blocks(np.frombuffer(data, dtype=np.uint8), w, explicit=True)


def test_corner_blocks_of_smoke_tensor():
    import pzinputs

    _check_blocks(pzinputs.corner_blocks(100).view(np.uint8), 16, explicit=True)


@pytest.mark.parametrize("w", [16, 32])
def test_ragged_tails(w):
    """Tensors of 0..300 bytes and around the chunk boundaries: round trip,
    header values and the stream length of the size model."""
    rng = np.random.default_rng(w + 1)
    base = np.maximum(rng.standard_normal(5000).astype(np.float32), 0).view(np.uint8)
    sizes = list(range(0, 301)) + [4095, 4096, 4097, 8191, 8192, 8193]
    for n in sizes:
        data = base[:n].copy()
        stream, tags, bits = oracle.compress(data, w, want_blocks=True)
        assert stream.size == size_model.stream_bytes(n, bits) if n else stream.size == 0
        assert oracle.decompress(stream, n, w).tobytes() == data.tobytes()
        C = (n + 4095) // 4096
        H = oracle.header_table(stream, n)
        assert H.size == C and stream.size == 2 * C + H.sum()
        # The padded last block is sized as a whole block with zero bytes.
        if n % 128:
            padded = np.zeros(((n + 127) // 128) * 128, np.uint8)
            padded[:n] = data
            model = size_model.candidate_sizes(padded, w)
            assert bits[-1] == 3 + model[-1].min()
