"""Run the oracle pins against a mutated oracle library (used by test_oracle_mutants).

usage: python _mutant_runner.py <mutated oracle.c> <output .so>
Exit status 0 means every pin still passed (the mutant survived)."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import pytest  # noqa: E402

oracle._SRC = sys.argv[1]
oracle._LIB = sys.argv[2]
oracle._lib = None
sys.exit(pytest.main([os.path.join(HERE, "test_oracle_pins.py"), "-x", "-q", "-p", "no:cacheprovider",
                      "-o", "addopts="]))
