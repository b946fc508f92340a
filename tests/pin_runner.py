"""Subprocess helper: run every oracle pin against the library at argv[1] and print
one line per pin, "PASS name" or "FAIL name". A mutant that crashes the process
counts as caught by the caller."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from oracle_pins import ALL_PINS  # noqa: E402

lib = oracle.load(sys.argv[1])
for pin in ALL_PINS:
    try:
        pin(lib)
        print("PASS", pin.__name__, flush=True)
    except Exception as e:  # AssertionError or a numeric error from a broken oracle
        print("FAIL", pin.__name__, type(e).__name__, flush=True)
