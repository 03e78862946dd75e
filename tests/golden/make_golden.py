"""Write the stored expected values that come from the oracle (not from the pages).

Calls only ``oracle/``. Run from the repository root: ``python tests/golden/make_golden.py``.
Output: ``nf4_codebook.txt`` - the 16 NF4 levels (fp16 values, ascending), built from
normal quantiles as described under "The formats" on the "INT4 and Low-Bit Inference"
page, with the end-probability reading documented in ``oracle/nf4.py``.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402


def main():
    c = oracle.nf4_codebook().astype(np.float64)
    with open(os.path.join(HERE, "nf4_codebook.txt"), "w") as f:
        f.write("# NF4 levels (fp16 values, ascending), written by tests/golden/make_golden.py\n")
        for v in c:
            f.write(f"{float(v)!r}\n")


if __name__ == "__main__":
    main()
