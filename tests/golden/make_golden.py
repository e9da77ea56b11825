"""Writes tests/golden/code_tables.txt from the CPU oracle (and nothing else).

The file is a regression guard for the oracle's fp32 code tables; the tables'
independent pins are the closed-form checks in tests/test_oracle_pins.py."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402


def main():
    with open(os.path.join(HERE, "code_tables.txt"), "w") as f:
        f.write("# fp32 bit patterns of the 4-bit code tables, code 0..15, written by make_golden.py\n")
        for name, t in (("nf4", O.nf4_table()), ("fp4", O.fp4_table())):
            f.write(name + " " + " ".join(f"{v:08x}" for v in t.view("uint32").tolist()) + "\n")


if __name__ == "__main__":
    main()
