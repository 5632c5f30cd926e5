"""Run every oracle pin against one oracle build and report each result on its own line.

Usage: python tests/_run_pins.py <path to an oracle shared library>
Prints 'PASS <pin>' or 'FAIL <pin>: <reason>' per pin; exits 0 unless the
process itself dies (a mutant that reads out of bounds may crash it).
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import _oracle_pins as pins  # noqa: E402


def main(lib):
    for pin in pins.ALL_PINS:
        try:
            pin(lib_path=lib)
            print(f"PASS {pin.__name__}", flush=True)
        except (AssertionError, ValueError) as e:
            print(f"FAIL {pin.__name__}: {str(e)[:120]}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
