"""Pins of the CPU oracle to what the PlaneZip paper fixes (no GPU).

* the code lengths of BPC's prefix code as sized in §III-A, exhaustively for
  small planes, and the completeness of the code (Kraft sum 1);
* hand-derived closed-form sizes of special blocks (tests/golden/closed_forms.txt);
* a hand-derived byte stream for an all-zero chunk;
* Table III's printed ratios for dropout masks and int64 indices
  (tests/golden/paper_values.txt);
* the geometric means of Table IV and Fig. 3 (pins the reading of the tables).
"""
import math
import os

import numpy as np
import pytest

import oracle
import pzinputs
from oracle import size_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _paper_values():
    out = {}
    with open(os.path.join(GOLDEN, "paper_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            out[parts[0]] = (float(parts[1]), float(parts[2]))
    return out


# --------------------------------------------------------------------------
# The plane coder
# --------------------------------------------------------------------------

# Code lengths stated in §III-A for the non-verbatim codes, and the 1-bit flag
# of a verbatim plane. A run code is 2 + R bits with R = log2(w).
def test_prefix_code_is_complete():
    lengths = [1, 2, 3, 5, 5, 5, 5]   # verbatim, run, lone zero, ones, pre-zero, pair, single
    assert sum(2.0 ** -n for n in lengths) == 1.0
    # Run codes are 6 bits for w = 16 and 7 for w = 32 (§III-A).
    assert 2 + int(math.log2(16)) == 6 and 2 + int(math.log2(32)) == 7


def _expected_plane_bits(P, L, R):
    """Code length of a stack of planes from the page's table, computed with
    Python integers (independent of both oracle implementations)."""
    K = len(P)
    X = [P[j] ^ (P[j + 1] if j + 1 < K else 0) for j in range(K)]
    pw = (L - 1).bit_length() if L >= 2 else 0
    bits = 0
    j = K - 1
    while j >= 0:
        if X[j] == 0:
            k = 0
            while j - k >= 0 and X[j - k] == 0:
                k += 1
            bits += 3 if k == 1 else 2 + R
            j -= k
            continue
        x = X[j]
        ones = bin(x).count("1")
        if x == (1 << L) - 1:
            bits += 5
        elif P[j] == 0:
            bits += 5
        elif ones == 2 and (x & (x >> 1)):
            bits += 5 + pw
        elif ones == 1:
            bits += 5 + pw
        else:
            bits += 1 + L
        j -= 1
    return bits


@pytest.mark.parametrize("L", list(range(0, 7)))
def test_plane_coder_exhaustive_two_planes(L):
    """Every pair of planes of width L <= 6: decode(code(P)) == P, all bits
    consumed, and the length follows the page's table."""
    R = 4
    for p1 in range(1 << L):
        for p0 in range(1 << L):
            P = [p0, p1]
            buf, nbits = oracle.code_planes(P, 2, L, R)
            assert nbits == _expected_plane_bits(P, L, R), (P, L)
            back, used = oracle.decode_planes(buf, nbits, 2, L, R)
            assert used == nbits
            assert [int(v) for v in back] == P


@pytest.mark.parametrize("L", list(range(7, 13)))
def test_plane_coder_exhaustive_one_plane(L):
    for R in (4, 5):
        for p in range(1 << L):
            buf, nbits = oracle.code_planes([p], 1, L, R)
            assert nbits == _expected_plane_bits([p], L, R)
            back, used = oracle.decode_planes(buf, nbits, 1, L, R)
            assert used == nbits and int(back[0]) == p


@pytest.mark.parametrize("K,L,R", [(17, 63, 4), (16, 64, 4), (16, 12, 4), (33, 31, 5), (32, 32, 5), (32, 9, 5)])
def test_plane_coder_random_stacks(K, L, R):
    """Random plane stacks with structure (zero runs, all-ones, single and
    paired ones) at the real plane counts and widths."""
    rng = np.random.default_rng(K * 100 + L)
    full = (1 << L) - 1
    for _ in range(300):
        P = []
        for _ in range(K):
            kind = rng.integers(0, 6)
            if kind == 0:
                v = 0
            elif kind == 1:
                v = full
            elif kind == 2 and L >= 1:
                v = 1 << int(rng.integers(0, L))
            elif kind == 3 and L >= 2:
                v = 3 << int(rng.integers(0, L - 1))
            elif kind == 4 and P:
                v = P[-1]
            else:
                v = int(rng.integers(0, 1 << 62)) & full
            P.append(v)
        buf, nbits = oracle.code_planes(P, K, L, R)
        assert nbits == _expected_plane_bits(P, L, R)
        back, used = oracle.decode_planes(buf, nbits, K, L, R)
        assert used == nbits and [int(v) for v in back] == P


def test_plane_code_bit_strings():
    """The stream-order code words of FORMAT.md §3 for one plane of width 8."""
    def bits_of(buf, n):
        return "".join(str((int(buf[t >> 3]) >> (t & 7)) & 1) for t in range(n))

    cases = [
        ([0, 0], "01" + "0000"),              # run of 2 planes, k-2 = 0 in 4 bits
        ([0], "001"),                          # one zero plane
        ([0xFF], "00000"),                     # all ones
        ([0b1, 0b1], "00011" + "000" + "001"),  # top: single one at 0; low: X = 0 -> lone zero
        ([0b1100], "00010" + "010"),           # two adjacent ones at p = 2 (LSB first)
        ([0b1000], "00011" + "110"),           # single one at p = 3
        ([0b10100101], "1" + "10100101"),      # verbatim, element 0 first
        ([0b10, 0], "00011" + "100" + "00001"),  # top single one at 1; low plane pre-XOR zero
        ([0, 0b10], "001" + "00011" + "100"),    # top zero plane; low single one at 1
    ]
    for P_top_first, expect in cases:
        P = list(reversed(P_top_first))
        buf, nbits = oracle.code_planes(P, len(P), 8, 4)
        assert bits_of(buf, nbits) == expect, (P_top_first, bits_of(buf, nbits), expect)


# --------------------------------------------------------------------------
# Closed forms and hand-derived streams
# --------------------------------------------------------------------------

def _pattern_block(w, pattern):
    kind, vals = pattern.split(":")
    vals = [int(v, 16) for v in vals.split(",")]
    n = 1024 // w
    dt = "<u2" if w == 16 else "<u4"
    if kind == "const":
        sym = np.full(n, vals[0], dtype=dt)
    else:
        sym = np.array(vals * (n // len(vals)), dtype=dt)
    return sym.view(np.uint8)


@pytest.mark.parametrize("row", _read_table("closed_forms.txt"), ids=lambda r: r[0])
def test_closed_form_sizes(row):
    name, w, pattern = row[0], int(row[1]), row[2]
    expect = [int(v) for v in row[3:8]]
    chosen = int(row[8])
    block = _pattern_block(w, pattern)
    assert list(oracle.block_sizes(block, w)) == expect
    assert list(size_model.candidate_sizes(block, w)[0]) == expect
    _, tags, bits = oracle.compress(block, w, want_blocks=True)
    assert int(tags[0]) == chosen
    assert int(bits[0]) == 3 + min(expect)


def test_zero_chunk_stream_bytes():
    """An all-zero 4 KiB BF16 chunk: 32 blocks of tag 2 (BX) followed by one
    run of 16 planes. Per block, in stream order: tag 2 = 0,1,0; run code 0,1;
    k-2 = 14 in 4 bits = 0,1,1,1. 288 bits = 36 bytes, header 36."""
    block_bits = [0, 1, 0, 0, 1, 0, 1, 1, 1]
    bits = block_bits * 32
    payload = bytearray(36)
    for t, b in enumerate(bits):
        payload[t >> 3] |= b << (t & 7)
    expect = bytes([36, 0]) + bytes(payload)
    got = oracle.compress(np.zeros(4096, np.uint8), 16).tobytes()
    assert got == expect
    assert len(got) == 38 and abs(4096 / 38 - 107.789) < 1e-3


def test_zero_chunk_fp32_ratio():
    s = oracle.compress(np.zeros(4096, np.uint8), 32)
    assert len(s) == 42          # 32 blocks * (3 + 7) bits = 40 bytes + header


def test_random_chunk_is_stored_raw():
    """Uniform random bits: every candidate exceeds 1024 bits, so blocks are
    RAW (3 + 1024 bits); 32 of them make 4108 bytes >= 4096, so the chunk is
    stored raw with H = 4096."""
    data = np.random.default_rng(11).integers(0, 256, 4096, dtype=np.uint8)
    s, tags, bits = oracle.compress(data, 16, want_blocks=True)
    assert (tags == 4).all() and (bits == 1027).all()
    assert len(s) == 4098 and int(s[0]) | (int(s[1]) << 8) == 4096
    assert s[2:].tobytes() == data.tobytes()


# --------------------------------------------------------------------------
# Table III worked examples
# --------------------------------------------------------------------------

def test_table3_dropout_mask():
    pv = _paper_values()
    t = pzinputs.dropout_mask(4 << 20)
    bx_only = oracle.compress(t.data, 32, codec_mask=1 << oracle.BX, tagged=False)
    planezip = oracle.compress(t.data, 32)
    r_bx = t.nbytes / bx_only.size
    r_pz = t.nbytes / planezip.size
    v, tol = pv["dropout_mask_bx"]
    assert abs(r_bx - v) <= tol, r_bx
    v, tol = pv["dropout_mask_planezip"]
    assert abs(r_pz - v) <= tol, r_pz


def test_table3_dropout_mask_rejects_reversed_xor():
    """The reverse XOR direction (bottom plane kept) would cost 5 more bits
    per block (four pre-XOR-zero codes and runs of 6 instead of three codes
    and a run of 7 at the top): 180 - 4*0.9**32*28 bits, giving about 5.79,
    outside the pin's tolerance. The oracle must not be at that value."""
    pv = _paper_values()
    reversed_bits = 180 - 4 * 0.9 ** 32 * 28
    per_block_bytes = reversed_bits / 8 + 2 / 32 + 0.44 / 32
    r_rev = 128 / per_block_bytes
    v, tol = pv["dropout_mask_bx"]
    assert abs(r_rev - v) > tol


def test_table3_int64_indices_zvc():
    pv = _paper_values()
    t = pzinputs.int64_indices(1 << 20)
    s = oracle.compress(t.data, 32, codec_mask=1 << oracle.ZVC, tagged=False)
    ratio = t.nbytes / s.size
    assert s.size == (t.nbytes // 4096) * (2 + 32 * (32 + 16 * 32) // 8)
    assert abs(ratio - 1024 / 544.5) < 1e-9
    v, tol = pv["indices_zvc"]
    assert abs(ratio - v) <= tol


def test_table_geometric_means():
    pv = _paper_values()
    bf16 = [1.88, 2.14, 1.40, 1.31, 1.97]
    fp32 = [1.74, 1.57, 1.50, 1.15, 1.11]
    g16 = math.exp(sum(map(math.log, bf16)) / 5)
    g32 = math.exp(sum(map(math.log, fp32)) / 5)
    v, tol = pv["geomean_bf16"]
    assert abs(g16 - v) <= tol
    v, tol = pv["geomean_fp32"]
    assert abs(g32 - v) <= tol
