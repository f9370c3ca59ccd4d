"""Builds the oracle's C library (``oracle/libpzref.so``) with the host compiler.

Test infrastructure only: see ``oracle/__init__.py``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(HERE, "pzref.c")
    out = os.path.join(HERE, "libpzref.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
           "-pthread", src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
