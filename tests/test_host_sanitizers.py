"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The CPU oracle (oracle/pzref.c) is rebuilt with both sanitizers and runs its
pin, brute-force and stream tests; the native predictor table
(lossless_bit_plane_amd/csrc/pz_predictor.cpp) is built alone with both and
runs the predictor tests' operation sequence against the plain table of
oracle/predictor.py, from one and from eight host threads. Any sanitizer
report aborts the run. (The swap engine's bookkeeping drives HIP streams and
events, so it is exercised by the GPU tests only.)"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime():
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("no host compiler")
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no AddressSanitizer runtime")
    return path


def _env(asan, **extra):
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1", **extra)
    return env


def _check(res):
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_oracle_under_sanitizers(tmp_path):
    asan = _runtime()
    lib = tmp_path / "libpzref_san.so"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread", *SAN,
                    os.path.join(ROOT, "oracle", "pzref.c"), "-o", str(lib)], check=True)
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_pins.py", "test_oracle_brute.py", "test_oracle_streams.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          "-k", "not gpt2", *tests], cwd=ROOT, capture_output=True, text=True,
                         env=_env(asan, PZREF_LIB=str(lib)), timeout=900)
    _check(res)
    assert " passed" in res.stdout


def test_predictor_under_sanitizers(tmp_path):
    asan = _runtime()
    lib = tmp_path / "libpzpred_san.so"
    subprocess.run(["g++", "-std=c++17", "-Wall", "-shared", "-fPIC", "-pthread", *SAN,
                    os.path.join(ROOT, "lossless_bit_plane_amd", "csrc", "pz_predictor.cpp"), "-o", str(lib)],
                   check=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_predictor.py"), str(lib)],
                         cwd=ROOT, capture_output=True, text=True, env=_env(asan), timeout=600)
    _check(res)
    assert "sanitized predictor: ok" in res.stdout
