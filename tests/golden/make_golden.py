"""Writes the frozen known-answer files under tests/golden/ from the oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import srhash  # noqa: E402


def write_sr_kat():
    cases = []
    for seed in (0, 1, 0xDEADBEEFCAFEF00D):
        for stream in (0, 1, 2, 3, 17):
            for idx in (0, 1, 2, 3, 1000, 1001, (1 << 32) - 1, 1 << 32, (1 << 33) + 5, 117440511):
                cases.append((seed, stream, idx))
    path = os.path.join(HERE, "sr_random16_kat.txt")
    with open(path, "w") as f:
        f.write("# seed stream element_index random16  (written by make_golden.py from oracle.srhash)\n")
        for seed, stream, idx in cases:
            r = srhash.random16(seed, stream, np.array([idx], dtype=np.uint64))[0]
            f.write(f"{seed} {stream} {idx} {int(r)}\n")


if __name__ == "__main__":
    write_sr_kat()
