"""Writes the stored expected values under tests/golden/ from the CPU oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def main():
    t = oracle.nf4_table()
    with open(os.path.join(HERE, "nf4_table.txt"), "w") as f:
        f.write("# NF4 code values (fp32) from oracle.nf4_table(): normal quantiles at evenly spaced\n")
        f.write("# probabilities, 7 negative / 0 / 8 positive, each side scaled to +-1 (the reading of the\n")
        f.write("# QLoRA blog's '1. NormalFloat' section).  Columns: code, fp32 bits (hex), value.\n")
        for i, v in enumerate(t):
            f.write(f"{i} {int(np.array(v).view(np.uint32)):08x} {float(v):.9g}\n")


if __name__ == "__main__":
    main()
