"""Write the stored expected values under tests/golden/ from the CPU oracle only.

Run from the repository root: python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def lesson_demo3():
    lines = [
        "# Reduction lesson page (03_shared_memory_sync_reduction.py), demo 3",
        "# (parallel reduction): float32 input x[i] = i mod 7 with 256-thread",
        "# blocks, n = 2^18 in the full run and 2^14 with --quick. 'expected' is",
        "# the float64 sum of that input, the value the page compares its block",
        "# partials against. Written by tests/golden/make_golden.py (oracle only).",
    ]
    for n in (1 << 18, 1 << 14):
        x = (np.arange(n) % 7).astype(np.float32)
        S, _ = oracle.sum_f32(x)
        lines.append(f"n={n} block=256 expected={int(S)}")
    with open(os.path.join(HERE, "lesson_demo3_mod7.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    lesson_demo3()
