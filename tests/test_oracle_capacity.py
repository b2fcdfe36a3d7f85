"""Pins of the oracle's expert-capacity formula (CPU only).

The capacity is max(min_capacity, ceil(k*T/E * capacity_factor)), evaluated in
IEEE double.  The pins: every worked capacity number the source pages print
(tests/golden/capacity_worked.json, each with its page and section), the five
workloads' capacities worked out by hand, the min_capacity floor and the
double-evaluation case where a non-dyadic factor lands just above an integer.
"""
import json
import os

import pytest

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "capacity_worked.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"T{c['T']}_E{c['E']}_cf{c['capacity_factor']}")
def test_pages_worked_capacity(case):
    k, T, E = case["k"], case["T"], case["E"]
    # assignments per expert, as the pages state it
    assert O.capacity(k, T, E, 1.0, 1, True) == case["per_expert"]
    assert O.capacity(k, T, E, case["capacity_factor"], 1, True) == case["capacity"]


@pytest.mark.parametrize("T,d,E,k,cf,want", [
    # tiny fp32 workload: 1*64/4 = 16, factor 1 -> 16
    (64, 32, 4, 1, 1.0, 16),
    # top-2, 8 experts: 2*4096/8 = 1024
    (4096, 512, 8, 2, 1.0, 1024),
    # top-2, 64 experts: 2*16384/64 = 512, x1.25 = 640
    (16384, 2048, 64, 2, 1.25, 640),
    # skewed, 16 experts: 2*32768/16 = 4096, x2 = 8192
    (32768, 4096, 16, 2, 2.0, 8192),
])
def test_workload_capacities(T, d, E, k, cf, want):
    assert O.capacity(k, T, E, cf, 4, True) == want


def test_min_capacity_floor():
    # ceil(1/64) = 1 < 4 -> the floor decides
    assert O.capacity(1, 1, 64, 1.0, 4, True) == 4
    assert O.capacity(2, 10, 64, 1.0, 0, True) == 1
    assert O.capacity(2, 0, 64, 1.0, 0, True) == 0
    assert O.capacity(2, 0, 64, 1.0, 7, True) == 7


def test_no_drop_has_no_capacity():
    assert O.capacity(2, 65536, 128, 1.0, 4, False) is None


def test_ceil_rounds_up_fractions():
    # 8/3 * 0.5 = 1.333.. -> 2
    assert O.capacity(2, 4, 3, 0.5, 1, True) == 2
    # 2*5/4 = 2.5 -> 3
    assert O.capacity(2, 5, 4, 1.0, 0, True) == 3


def test_double_evaluation_of_nondyadic_factor():
    # k*T/E = 50 exactly, but 50 * 1.1 in IEEE double is 55.00000000000001,
    # so the ceiling is 56, not the decimal 55.  The library evaluates the same
    # double expression; the ABI test checks that it agrees.
    assert 50.0 * 1.1 > 55.0
    assert O.capacity(2, 100, 4, 1.1, 0, True) == 56
