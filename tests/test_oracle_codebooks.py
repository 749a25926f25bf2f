"""Pins for the oracle's mcg and 3INST procedural codebooks.

Source: "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture item 5
(the three procedural codebooks; counts of distinct levels printed for each),
and the published three-instruction (3INST) decoder of the QTIP trellis codes.

The printed counts (tests/golden/pages_figures.json) are fingerprints of the
whole construction: a different multiplier, increment, mask, xor pattern or a
binary32 instead of binary16 sum of the halves changes them.  A second,
independent evaluation of individual states (halves decoded from their bit
fields into exact rationals, the sum rounded by a nearest search over every
finite binary16 value) pins the mask / xor / sum / rounding steps.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _figures():
    with open(os.path.join(GOLDEN, "pages_figures.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["mcg", "3inst"])
def test_distinct_level_count_is_the_printed_one(name):
    levels = oracle.CODEBOOKS[name]()
    assert levels.dtype == np.float16 and levels.shape == (65536,)
    assert len(np.unique(levels)) == _figures()[name]["distinct_levels"]


def test_neighbouring_constructions_give_other_counts():
    # the count is sensitive: a binary32 sum of the halves, or another odd
    # multiplier, does not reproduce it
    s = np.arange(65536, dtype=np.uint64)
    words = (s * np.uint64(oracle.reference.MCG_MULTIPLIER)) & np.uint64(0xFFFFFFFF)
    m = (words & np.uint64(0x8FFF8FFF)) ^ np.uint64(0x3B603B60)
    lo = (m & np.uint64(0xFFFF)).astype(np.uint16).view(np.float16).astype(np.float32)
    hi = (m >> np.uint64(16)).astype(np.uint16).view(np.float16).astype(np.float32)
    assert len(np.unique(lo + hi)) != 10746
    start = oracle.reference.MCG_SCAN_START
    other = oracle.reference._halves_sum_fp16((s * np.uint64(start)) & np.uint64(0xFFFFFFFF))
    assert len(np.unique(other)) != 10746


def test_mcg_multiplier_is_the_first_hit_of_the_scan():
    # the pages print the count but no multiplier: the reading takes the first
    # odd multiplier from the golden-ratio constant up that reproduces it
    a, scanned = oracle.reference.mcg_multiplier_scan()
    assert a == oracle.reference.MCG_MULTIPLIER == 0x9E378FED
    assert scanned == 2847
    assert oracle.reference.MCG_SCAN_START == oracle.MUL1_MULTIPLIER


def _half_value(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    assert 0 < e < 31
    return sign * Fraction(1024 + f, 1024) * Fraction(2) ** (e - 15)


_ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
_FINITE_BITS = np.flatnonzero(np.isfinite(_ALL))
_FINITE_VALS = _ALL[_FINITE_BITS].astype(np.float64)


def _nearest_fp16_bits(x: Fraction) -> int:
    """Nearest finite binary16 to x, ties to the even bit pattern (brute force)."""
    d = np.abs(_FINITE_VALS - float(x))
    cand = _FINITE_BITS[d <= d.min() * (1 + 1e-12) + 1e-300]
    best = min(cand, key=lambda b: (abs(Fraction(float(_ALL[b])) - x), b & 1))
    return int(best)


def _word(name, s):
    if name == "mcg":
        return (oracle.reference.MCG_MULTIPLIER * s) % 2 ** 32
    return (oracle.reference.INST3_A * s + oracle.reference.INST3_B) % 2 ** 32


@pytest.mark.parametrize("name", ["mcg", "3inst"])
def test_individual_states_by_exact_arithmetic(name):
    levels = oracle.CODEBOOKS[name]().view(np.uint16)
    rng = np.random.Generator(np.random.PCG64(77))
    states = [0, 1, 2, 255, 256, 32767, 32768, 65535] + rng.integers(0, 65536, 40).tolist()
    for s in states:
        m = (_word(name, s) & 0x8FFF8FFF) ^ 0x3B603B60
        a, b = _half_value(m & 0xFFFF), _half_value(m >> 16)
        # every half has exponent field 12..15: magnitude in [1/8, 2)
        assert Fraction(1, 8) <= abs(a) < 2 and Fraction(1, 8) <= abs(b) < 2
        assert levels[s] == _nearest_fp16_bits(a + b), (name, s)


def test_mcg_state_zero_closed_form():
    # state 0: the word is 0, both halves are 0x3B60 = 0.921875, the level 1.84375
    assert float(oracle.mcg_levels_fp16()[0]) == 1.84375


@pytest.mark.parametrize("name", ["mcg", "3inst"])
def test_levels_are_bounded_and_near_unit_scale(name):
    v = oracle.CODEBOOKS[name]().astype(np.float64)
    assert np.all(np.abs(v) < 4.0)
    assert 1.1 < v.std() < 1.4 and abs(v.mean()) < 0.05
