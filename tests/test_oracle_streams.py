"""Whole-stream checks of the CPU oracle on the synthetic workloads (no GPU).

* round trip of every workload tensor (the smoke tensor in full, block
  samples of the larger ones) and of the edge tensors;
* the numpy size model equals the C encoder's bit counts for every sampled
  block, and the stream length equals 2C plus the padded chunk lengths;
* corrupt streams (FORMAT.md §6) are rejected;
* single-codec variants and the threaded driver.
"""
import numpy as np
import pytest

import oracle
import pzinputs
from oracle import size_model


def _roundtrip_with_model(data, w):
    stream, tags, bits = oracle.compress(data, w, want_blocks=True)
    n = data.size
    assert stream.size == size_model.stream_bytes(n, bits)
    assert oracle.decompress(stream, n, w).tobytes() == data.tobytes()
    return stream, tags, bits


def test_relu_smoke_full(workload_tensors):
    (t,) = workload_tensors("relu-smoke")
    assert t.nbytes == 1056768
    stream, tags, bits = _roundtrip_with_model(t.data, 16)
    blocks = t.data.reshape(-1, 128)
    model = size_model.candidate_sizes(blocks, 16)
    np.testing.assert_array_equal(oracle.blocks_sizes(blocks, 16), model)
    np.testing.assert_array_equal(tags, size_model.select(model))
    # ReLU data is half zeros, so ZBX occurs; the corner blocks reach DBX, BX
    # and RAW. (ZVC wins only on very sparse blocks, which the brute-force
    # tests cover.)
    assert {1, 2, 3, 4} <= set(int(v) for v in np.unique(tags))


@pytest.mark.parametrize("k,name", [(2, "cnn-fp32"), (3, "gpt2-small"), (4, "vit-layernorm"), (5, "gpt2-xl")])
def test_workload_block_samples(workload_tensors, k, name):
    """Two implementations agree on 3,000 sampled blocks of every tensor, and
    sampled whole chunks round-trip."""
    for i, t in enumerate(workload_tensors(name)):
        blocks = pzinputs.sample_blocks(t, 3000, seed=k * 10 + i)
        model = size_model.candidate_sizes(blocks, t.elem_bits)
        np.testing.assert_array_equal(oracle.blocks_sizes(blocks, t.elem_bits), model)
        rng = np.random.default_rng(k)
        C = t.nbytes // 4096
        for c in rng.choice(C, size=8, replace=False):
            chunk = t.data[4096 * c: 4096 * (c + 1)]
            _roundtrip_with_model(chunk, t.elem_bits)


def test_edge_tensors():
    for t in pzinputs.edge_tensors():
        _roundtrip_with_model(t.data, t.elem_bits)


def test_threaded_driver_matches(workload_tensors):
    (t,) = workload_tensors("relu-smoke")
    s1 = oracle.compress(t.data, 16)
    s4 = oracle.compress(t.data, 16, threads=4)
    assert s1.tobytes() == s4.tobytes()
    assert oracle.decompress(s4, t.nbytes, 16, threads=3).tobytes() == t.data.tobytes()


@pytest.mark.parametrize("cand", [0, 1, 2, 3, 4])
def test_single_codec_variants(workload_tensors, cand):
    """One fixed encoding, no tag (the paper's per-codec columns)."""
    (t,) = workload_tensors("relu-smoke")
    data = t.data[: 64 * 4096]
    mask = 1 << cand
    s = oracle.compress(data, 16, codec_mask=mask, tagged=False)
    back = oracle.decompress(s, data.size, 16, codec_mask=mask, tagged=False)
    assert back.tobytes() == data.tobytes()
    model = size_model.candidate_sizes(data.reshape(-1, 128), 16)
    assert s.size == size_model.stream_bytes(data.size, model[:, cand])


def test_bf16_as_32_bit_symbols(workload_tensors):
    """BF16 data coded with w = 32 (§V-A ablation) round-trips and compresses
    less than with w = 16 on ReLU data."""
    (t,) = workload_tensors("relu-smoke")
    s16 = oracle.compress(t.data, 16)
    s32, _, _ = _roundtrip_with_model(t.data, 32)
    assert s32.size > s16.size


# --------------------------------------------------------------------------
# Corrupt streams (FORMAT.md §6)
# --------------------------------------------------------------------------

def _good_stream():
    (t,) = [pzinputs.relu_smoke()[0]]
    data = t.data[: 3 * 4096 + 1000].copy()
    return data, oracle.compress(data, 16)


def _status(stream, n):
    return oracle.decompress_status(stream, n, 16)


def test_corrupt_total_length():
    data, s = _good_stream()
    assert _status(s, data.size) == oracle.OK
    assert _status(s[:-1], data.size) == oracle.ECORRUPT
    assert _status(np.concatenate([s, np.zeros(1, np.uint8)]), data.size) == oracle.ECORRUPT
    assert _status(s[:5], data.size) == oracle.ECORRUPT


def test_corrupt_header_above_raw_length():
    data = np.zeros(4096, np.uint8)
    s = bytearray(2 + 4097)
    s[0], s[1] = 4097 & 0xFF, 4097 >> 8
    assert _status(np.frombuffer(bytes(s), np.uint8), 4096) == oracle.ECORRUPT


def _stream_from_bits(bits, raw_len):
    nbytes = (len(bits) + 7) // 8
    payload = bytearray(nbytes)
    for t, b in enumerate(bits):
        payload[t >> 3] |= b << (t & 7)
    return np.frombuffer(bytes([nbytes & 0xFF, nbytes >> 8]) + bytes(payload), np.uint8)


def _field(v, n):
    return [(v >> i) & 1 for i in range(n)]


def test_corrupt_tags():
    for tag in (5, 6, 7):
        s = _stream_from_bits(_field(tag, 3) + [0] * 20, 128)
        assert _status(s, 128) == oracle.ECORRUPT


def test_zero_run_overflow():
    # BX block (tag 2) whose first code is a run of 17 > 16 planes.
    bits = _field(2, 3) + [0, 1] + _field(15, 4)
    assert _status(_stream_from_bits(bits, 128), 128) == oracle.ECORRUPT
    # A run of exactly 16 planes is a valid all-zero block.
    bits = _field(2, 3) + [0, 1] + _field(14, 4)
    assert _status(_stream_from_bits(bits, 128), 128) == oracle.OK


def test_position_out_of_range():
    # ZBX block with n = 5 (PW = 3): a single one at p = 5 > L-1, and a pair at
    # p = 4 > L-2, are corrupt; p = 4 and p = 3 are fine.
    mask = [1] * 5 + [0] * 59
    def zbx(code, p):
        return _field(3, 3) + mask + code + _field(p, 3) + [0, 1] + _field(13, 4)
    single, pair = [0, 0, 0, 1, 1], [0, 0, 0, 1, 0]
    assert _status(_stream_from_bits(zbx(single, 5), 128), 128) == oracle.ECORRUPT
    assert _status(_stream_from_bits(zbx(pair, 4), 128), 128) == oracle.ECORRUPT
    assert _status(_stream_from_bits(zbx(single, 4), 128), 128) == oracle.OK
    assert _status(_stream_from_bits(zbx(pair, 3), 128), 128) == oracle.OK


def test_parse_overrun_and_padding():
    good = _field(2, 3) + [0, 1] + _field(14, 4)           # 9 bits -> 2 bytes
    s = _stream_from_bits(good, 128)
    assert _status(s, 128) == oracle.OK
    # Non-zero padding bit.
    bad = bytearray(s.tobytes())
    bad[3] |= 0x80
    assert _status(np.frombuffer(bytes(bad), np.uint8), 128) == oracle.ECORRUPT
    # A header one byte too long leaves a whole unused byte.
    longer = np.frombuffer(bytes([3, 0]) + s[2:].tobytes() + b"\x00", np.uint8)
    assert _status(longer, 128) == oracle.ECORRUPT
    # A header too short makes the parse run past the payload.
    shorter = np.frombuffer(bytes([1, 0]) + s[2:3].tobytes(), np.uint8)
    assert _status(shorter, 128) == oracle.ECORRUPT
