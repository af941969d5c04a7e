"""Writes the oracle-derived regression fixtures in this folder.

Calls only the oracle.  Run from the repository root:
    python tests/golden/make_golden.py
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import splitmix  # noqa: E402


def main():
    with open(os.path.join(HERE, "rht_signs.txt"), "w") as f:
        f.write("# First 64 RHT signs (1 = minus) for seeds 0 and 1, frozen from the\n"
                "# oracle's SplitMix64 key layout; a regression vector for both\n"
                "# independent implementations.  Written by make_golden.py.\n")
        for seed in (0, 1):
            s = splitmix.rht_signs(seed, 64)
            f.write("%d %s\n" % (seed, "".join("1" if v < 0 else "0" for v in s)))


if __name__ == "__main__":
    main()
