"""Run every oracle pin against one build of the oracle library.

Usage: python -m tests.run_pins <path to liboracle build>
Exit status: 0 if every pin holds, 1 if any pin fails.
"""
import sys

import oracle
from tests import oracle_pins


def main(path):
    orc = oracle.Oracle(path)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as exc:  # a pin that raises (assert or error) has caught the build
            failed.append(f"{pin.__name__}: {type(exc).__name__}")
    for f in failed:
        print("FAIL", f)
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
