"""The oracle against its pins (library routines, closed forms, brute
force, invariants); see tests/oracle_pins.py for what each one checks."""

import os, sys
import pytest
sys.path.insert(0, os.path.dirname(__file__))

import oracle.nosa_oracle as O
from oracle_pins import ALL_CHECKS, check_select_bruteforce


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(O)


def test_select_bruteforce_with_ties():
    check_select_bruteforce(O, seed=40, trials=300, ties=True)
