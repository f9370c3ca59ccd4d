"""Per-tensor compressibility predictor of the PlaneZip runtime, written out
plainly (PlaneZip paper §III-B "Compressibility Predictor").

TEST INFRASTRUCTURE ONLY: it checks the native table of the library; only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it.

What the pages fix: a saved tensor is identified by a signature (its
producing operator's position in the operator sequence and its output slot);
the runtime keeps one compression ratio per signature; every reported size
overwrites the entry; a signature without a measurement is taken to have a
ratio of one. Readings: the entry keeps the measured (raw, compressed) pair,
and a prediction for raw bytes m is ceil(m * compressed / raw).
"""
from __future__ import annotations


class RatioTable:
    def __init__(self):
        self.entries = {}

    def update(self, sig: int, raw_bytes: int, comp_bytes: int) -> None:
        self.entries[sig] = (raw_bytes, comp_bytes)

    def predict(self, sig: int, raw_bytes: int):
        """(predicted compressed bytes, measured?)."""
        if sig not in self.entries:
            return raw_bytes, False
        raw, comp = self.entries[sig]
        return -(-(raw_bytes * comp) // raw), True


def wire_error(predicted, actual) -> float:
    """Prediction error as a share of the wire bytes, the measure of the
    paper's Table IV: sum |predicted - actual| / sum actual."""
    num = sum(abs(p - a) for p, a in zip(predicted, actual))
    den = sum(actual)
    return num / den if den else 0.0
