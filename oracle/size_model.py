"""Vectorized size model of the five PlaneZip candidates (numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The PlaneZip paper's validation paragraph (§III-A) describes two
implementations of every encoder: a vectorized size model and a bit-exact
encoder and decoder, whose bit counts agree exactly. This module is the
first kind, written independently of ``pzref.c``: it never emits a bit. It
builds each block's bit-planes as boolean arrays and sizes them with the code
lengths that §III-A gives for BPC's prefix code:

* 3 bits for a lone all-zero plane, 2+R bits for a run of them (R = log2 w,
  so 6 bits for w = 16 and 7 for w = 32);
* 5 bits when the XORed plane is all ones or the plane before the XOR is 0;
* 5 bits plus a position when the plane holds a single 1 or a 1-1 pair;
* 1 bit plus the plane verbatim otherwise;

with the readings of FORMAT.md (top plane kept, codes in top-down order,
first matching rule wins, position width ceil(log2 L)).
"""
from __future__ import annotations

import numpy as np

ZVC, DBX, BX, ZBX, RAW = 0, 1, 2, 3, 4


def _symbols(blocks_u8: np.ndarray, w: int) -> np.ndarray:
    b = np.ascontiguousarray(blocks_u8, dtype=np.uint8).reshape(-1, 128)
    dt = "<u2" if w == 16 else "<u4"
    return b.view(dt).astype(np.int64)  # (nb, N)


def _bits(values: np.ndarray, nbits: int) -> np.ndarray:
    """(nb, L) integers -> (nb, nbits, L) booleans: [b, j, k] = bit j of values[b, k]."""
    j = np.arange(nbits, dtype=np.int64)[None, :, None]
    return ((values[:, None, :] >> j) & 1).astype(bool)


def _position_width(L: np.ndarray) -> np.ndarray:
    L = np.asarray(L, dtype=np.int64)
    pw = np.zeros_like(L)
    for p in range(1, 8):
        pw = np.where((L >= 2) & ((1 << (p - 1)) < L), p, pw)
    return pw


def plane_code_bits(P: np.ndarray, valid: np.ndarray, L: np.ndarray, R: int) -> np.ndarray:
    """Total code length of a stack of planes.

    P: (nb, K, Lmax) booleans, plane j = P[:, j, :], element k = P[:, :, k].
    valid: (nb, Lmax) booleans, which elements belong to the plane (k < L).
    L: (nb,) plane widths. Returns (nb,) bit counts.
    """
    nb, K, _ = P.shape
    P = P & valid[:, None, :]
    above = np.concatenate([P[:, 1:, :], np.zeros_like(P[:, :1, :])], axis=1)
    X = P ^ above
    count = X.sum(axis=2)                                   # ones per XORed plane
    zero = count == 0
    ones = (count == L[:, None]) & (L[:, None] > 0)
    pre_zero = ~P.any(axis=2)
    adjacent = (X[:, :, :-1] & X[:, :, 1:]).any(axis=2)
    pair = (count == 2) & adjacent
    single = count == 1
    pw = _position_width(L)[:, None]
    verbatim = 1 + L[:, None]
    nz_len = np.where(ones, 5,
             np.where(pre_zero, 5,
             np.where(pair, 5 + pw,
             np.where(single, 5 + pw, verbatim))))
    nonzero_bits = np.where(zero, 0, nz_len).sum(axis=1)

    # Maximal runs of zero planes, read in the top-down emission order.
    up = np.concatenate([zero[:, 1:], np.zeros((nb, 1), bool)], axis=1)    # zero[j+1]
    down = np.concatenate([np.zeros((nb, 1), bool), zero[:, :-1]], axis=1)  # zero[j-1]
    starts = zero & ~up
    lone = starts & ~down
    runs = starts.sum(axis=1)
    lone_runs = lone.sum(axis=1)
    run_bits = 3 * lone_runs + (2 + R) * (runs - lone_runs)
    return nonzero_bits + run_bits


def candidate_sizes(blocks_u8: np.ndarray, w: int, batch: int = 8192) -> np.ndarray:
    """(nblocks, 5) payload bit counts: ZVC, DBX, BX, ZBX, RAW."""
    s_all = _symbols(blocks_u8, w)
    out = np.zeros((s_all.shape[0], 5), dtype=np.int64)
    for lo in range(0, s_all.shape[0], batch):
        out[lo:lo + batch] = _sizes(s_all[lo:lo + batch], w)
    return out


def _sizes(s: np.ndarray, w: int) -> np.ndarray:
    nb, N = s.shape
    R = int(np.log2(w))
    res = np.zeros((nb, 5), dtype=np.int64)
    nonzero = s != 0
    n = nonzero.sum(axis=1)

    # ZVC: mask plus the surviving symbols.
    res[:, ZVC] = N + w * n

    # BX: w planes of the N symbols.
    full = np.ones((nb, N), bool)
    res[:, BX] = plane_code_bits(_bits(s, w), full, np.full(nb, N), R)

    # DBX: the first symbol, then the w+1 planes of the N-1 neighbour
    # differences written as (w+1)-bit two's complement numbers.
    d = (s[:, 1:] - s[:, :-1]) & ((1 << (w + 1)) - 1)
    res[:, DBX] = w + plane_code_bits(_bits(d, w + 1), np.ones((nb, N - 1), bool),
                                      np.full(nb, N - 1), R)

    # ZBX: mask, then BX over the non-zero symbols moved to the front.
    order = np.argsort(~nonzero, axis=1, kind="stable")
    packed = np.take_along_axis(s, order, axis=1)
    valid = np.arange(N)[None, :] < n[:, None]
    packed = np.where(valid, packed, 0)
    res[:, ZBX] = N + plane_code_bits(_bits(packed, w), valid, n, R)

    res[:, RAW] = 1024
    return res


def select(sizes: np.ndarray, codec_mask: int = 0x1F) -> np.ndarray:
    """Chosen tag per block: the smallest allowed candidate, ties to the lowest tag."""
    big = np.iinfo(np.int64).max
    allowed = np.array([(codec_mask >> t) & 1 for t in range(5)], bool)
    masked = np.where(allowed[None, :], sizes, big)
    return np.argmin(masked, axis=1)  # argmin returns the first of equal minima


def stream_bytes(raw_bytes: int, block_bits: np.ndarray) -> int:
    """Stream size from per-block coded bits (tag included): 2C + sum over
    chunks of the padded length, or the raw length of a chunk that would grow."""
    C = (raw_bytes + 4095) // 4096
    total = 2 * C
    for c in range(C):
        raw_len = min(4096, raw_bytes - 4096 * c)
        nb = (raw_len + 127) // 128
        bits = int(block_bits[32 * c: 32 * c + nb].sum())
        L = (bits + 7) // 8
        total += raw_len if L >= raw_len else L
    return total
