"""Writes the stored NF4 level table from the oracle (run by hand; calls only oracle/).

Output: tests/golden/nf4_levels.txt, one level per line as the fp32 bit
pattern in hex and the decimal value.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import nf4  # noqa: E402


def main():
    levels = nf4.nf4_levels()
    path = os.path.join(HERE, "nf4_levels.txt")
    with open(path, "w") as f:
        f.write("# NF4 level table (fp32), written by tests/golden/make_golden.py from\n")
        f.write("# oracle.nf4.nf4_levels(): asymmetric normal-quantile construction with\n")
        f.write("# delta = ((1 - 1/30) + (1 - 1/32)) / 2. Columns: index, fp32 bits (hex), value.\n")
        for i, v in enumerate(levels):
            f.write(f"{i} {int(levels[i:i+1].view('uint32')[0]):08x} {float(v):.9g}\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
