"""Per-tensor compressibility predictor (the ``pz_predictor_*`` calls of the C
ABI; PlaneZip paper §III-B "Compressibility Predictor").

Argument marshalling only: the table lives in the native library.
"""
from __future__ import annotations

import ctypes

from ._lib import check, lib


def signature(op_index: int, output_slot: int) -> int:
    """PZ_SIGNATURE: the producing operator's position in the operator
    sequence and its output slot."""
    return ((op_index << 16) | (output_slot & 0xFFFF)) & 0xFFFFFFFFFFFFFFFF


def pz_predictor_create(capacity: int):
    h = lib.pz_predictor_create(capacity)
    if not h:
        raise ValueError(f"pz_predictor_create({capacity}) failed")
    return h


def pz_predictor_destroy(handle) -> None:
    lib.pz_predictor_destroy(handle)


def pz_predictor_update(handle, sig: int, raw_bytes: int, comp_bytes: int) -> None:
    check(lib.pz_predictor_update(handle, sig, raw_bytes, comp_bytes), "pz_predictor_update")


def pz_predictor_predict(handle, sig: int, raw_bytes: int):
    """(predicted compressed bytes, whether the signature has a measurement)."""
    out = ctypes.c_uint64(0)
    measured = ctypes.c_int(0)
    check(lib.pz_predictor_predict(handle, sig, raw_bytes, ctypes.byref(out), ctypes.byref(measured)),
          "pz_predictor_predict")
    return int(out.value), bool(measured.value)


def pz_predictor_entries(handle) -> int:
    return int(lib.pz_predictor_entries(handle))


def pz_predictor_clear(handle) -> None:
    lib.pz_predictor_clear(handle)


def transfer_time(raw_bytes: int, ratio: float, link_bytes_per_s: float, engine_bytes_per_s: float) -> float:
    """pz_transfer_time: seconds one swap of the tensor occupies a copy queue
    (PlaneZip §III-C, Eq. 2), min(m/g, max(m/(c g), m/B))."""
    x = lib.pz_transfer_time(raw_bytes, ratio, link_bytes_per_s, engine_bytes_per_s)
    if x < 0:
        raise ValueError("pz_transfer_time: ratio and rates must be positive and finite")
    return float(x)


class Predictor:
    """Owns one table; the methods are the calls above."""

    def __init__(self, capacity: int = 512):
        self.handle = pz_predictor_create(capacity)

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            pz_predictor_destroy(h)

    def update(self, sig: int, raw_bytes: int, comp_bytes: int) -> None:
        pz_predictor_update(self.handle, sig, raw_bytes, comp_bytes)

    def predict(self, sig: int, raw_bytes: int):
        return pz_predictor_predict(self.handle, sig, raw_bytes)

    def __len__(self) -> int:
        return pz_predictor_entries(self.handle)

    def clear(self) -> None:
        pz_predictor_clear(self.handle)
