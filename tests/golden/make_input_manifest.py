"""Writes input_sha256.txt: the SHA-256 of every tensor of every synthetic
workload, as pzinputs generates it (seeded generators, no codec arithmetic).
The bench checks its inputs against this manifest, and a CPU test checks that
the generators still produce these bytes.

    python3 tests/golden/make_input_manifest.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import pzinputs  # noqa: E402


def main():
    lines = ["# SHA-256 of the synthetic workloads' tensors (pzinputs), written by",
             "# tests/golden/make_input_manifest.py.",
             "#",
             "# workload  tensor  bytes  sha256"]
    for name in pzinputs.WORKLOADS:
        for t in pzinputs.workload(name):
            lines.append(f"{name}  {t.name}  {t.nbytes}  {t.sha256()}")
            print(lines[-1], flush=True)
    with open(os.path.join(HERE, "input_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
