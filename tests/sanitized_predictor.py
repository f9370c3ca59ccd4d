"""Driver for tests/test_host_sanitizers.py (not collected): runs the native
predictor table, built alone with AddressSanitizer and UBSan, through the
operation sequence of the predictor tests against the plain table of
oracle/predictor.py. Usage: python sanitized_predictor.py LIBRARY"""
import ctypes
import os
import random
import sys
import threading

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from oracle.predictor import RatioTable  # noqa: E402

OK, INVALID, INSUFFICIENT = 0, 1, 2


def main(path):
    lib = ctypes.CDLL(path)
    vp, u64, sz, i = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_int
    lib.pz_predictor_create.argtypes = [sz]
    lib.pz_predictor_create.restype = vp
    lib.pz_predictor_destroy.argtypes = [vp]
    lib.pz_predictor_destroy.restype = None
    lib.pz_predictor_update.argtypes = [vp, u64, u64, u64]
    lib.pz_predictor_update.restype = i
    lib.pz_predictor_predict.argtypes = [vp, u64, u64, ctypes.POINTER(u64), ctypes.POINTER(i)]
    lib.pz_predictor_predict.restype = i
    lib.pz_predictor_entries.argtypes = [vp]
    lib.pz_predictor_entries.restype = sz
    lib.pz_predictor_clear.argtypes = [vp]
    lib.pz_predictor_clear.restype = None

    def predict(t, sig, raw):
        out, found = u64(), i()
        st = lib.pz_predictor_predict(t, sig, raw, ctypes.byref(out), ctypes.byref(found))
        return st, out.value, bool(found.value)

    # Random sequence against the plain table.
    rng = random.Random(11)
    t = lib.pz_predictor_create(512)
    ref = RatioTable()
    sigs = [(op << 16) | slot for op in range(150) for slot in range(2)]
    for step in range(6000):
        sig = rng.choice(sigs)
        raw = rng.choice([1, 2, 4095, 4096, 4097, rng.randrange(1, 1 << 20), rng.randrange(1, 1 << 40)])
        if rng.random() < 0.4:
            max_comp = 2 * ((raw + 4095) // 4096) + raw
            comp = rng.choice([1, max_comp, rng.randrange(1, max_comp + 1)])
            assert lib.pz_predictor_update(t, sig, raw, comp) == OK
            ref.update(sig, raw, comp)
        else:
            st, got, found = predict(t, sig, raw)
            assert st == OK and (got, found) == ref.predict(sig, raw), step
    assert lib.pz_predictor_entries(t) == len(ref.entries)
    lib.pz_predictor_destroy(t)

    # Capacity, invalid sizes, overflow, clear.
    t = lib.pz_predictor_create(4)
    for k in range(4):
        assert lib.pz_predictor_update(t, k << 16, 4096, 100 + k) == OK
    assert lib.pz_predictor_update(t, 99 << 16, 4096, 100) == INSUFFICIENT
    for raw, comp in [(0, 1), (10, 0), (4096, 4099), (1, 4)]:
        assert lib.pz_predictor_update(t, 1 << 16, raw, comp) == INVALID
    assert lib.pz_predictor_update(t, 1 << 16, 1, 3) == OK
    assert predict(t, 1 << 16, 1 << 63)[0] != OK
    lib.pz_predictor_clear(t)
    assert lib.pz_predictor_entries(t) == 0
    lib.pz_predictor_destroy(t)
    assert not lib.pz_predictor_create(0)

    # Eight host threads on one table.
    t = lib.pz_predictor_create(1024)
    last = {}

    def worker(k):
        r = random.Random(k)
        for _ in range(2000):
            sig = (k * 100 + r.randrange(100)) << 16
            comp = r.randrange(1, 4099)
            assert lib.pz_predictor_update(t, sig, 4096, comp) == OK
            last[sig] = comp
            predict(t, r.randrange(800) << 16, 4096)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert lib.pz_predictor_entries(t) == len(last)
    for sig, comp in last.items():
        assert predict(t, sig, 4096) == (OK, comp, True)
    lib.pz_predictor_destroy(t)
    print("sanitized predictor: ok")


if __name__ == "__main__":
    main(sys.argv[1])
