"""Writes the stored expected values that come from the oracle (not from the
pages).  It calls only oracle/.  Run from the repo root:

    python tests/golden/make_golden.py

nf4_levels_fp32.txt: the canonical fp32 NF4 levels (bit patterns), i.e. the
oracle's evaluation of the ultralytics "QLoRA" construction in torch fp32.  It
is a regression fixture guarding the oracle against library drift; the levels
themselves are pinned to mpmath, to the pages' invariants and to the page's
printed MSE figures in tests/test_oracle_codebook.py.
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.codebook import nf4_levels  # noqa: E402


def main():
    lv = nf4_levels()
    with open(os.path.join(HERE, "nf4_levels_fp32.txt"), "w") as f:
        f.write("# NF4 levels, fp32 bit patterns, ascending (index: hex value).\n")
        f.write("# Written by tests/golden/make_golden.py from oracle.codebook.nf4_levels().\n")
        for j, v in enumerate(lv.view("uint32")):
            f.write(f"{j}: {int(v):08x} {float(lv[j]):+.10f}\n")


if __name__ == "__main__":
    main()
