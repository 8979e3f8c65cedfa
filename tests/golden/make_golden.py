"""Writes the stored values under tests/golden/ that come from the oracle.

Calls only ``oracle/``.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import lbq_oracle as O  # noqa: E402


def main():
    c = O.nf4_codebook()
    with open(os.path.join(HERE, "nf4_codebook.txt"), "w") as f:
        f.write("# NF4 levels as fp32 bit patterns (hex) and decimal, ascending.\n")
        f.write("# Written by tests/golden/make_golden.py from oracle.nf4_codebook():\n")
        f.write("# normal quantiles at evenly spaced probabilities, exact zero, scaled to [-1, 1]\n")
        f.write("# (\"QLoRA技术在量化微调中的应用\", section QLoRA技术原理: NF4 suits normally\n")
        f.write("# distributed weights; the exact construction is a reading of that remark).\n")
        for v in c:
            f.write("%08x %.9g\n" % (int(v.view("uint32")), float(v)))


if __name__ == "__main__":
    main()
