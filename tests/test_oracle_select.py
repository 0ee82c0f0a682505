"""Pins for oracle.select (history frame selection).

The power-spaced policy is pinned by the worked example printed on the page
("Hy-Nomas: an 8.6B world model ...", section "The 4090 preset"; stored in
tests/golden/power_select_T360.txt) and by invariants that follow from the
equation: N picks, strictly increasing, always the oldest and newest frame, all
frames when the budget covers the history. ANCHOR_RECENT is pinned by a
per-frame brute-force membership rule.
"""

import os

import numpy as np
import pytest

from oracle import select

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "power_select_T360.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            head, frames = line.split(":")
            T, B, g = head.split()
            rows.append((int(T), int(B), float(g), [int(x) for x in frames.split()]))
    return rows


def test_power_matches_printed_example():
    rows = _golden_rows()
    assert rows
    for T, B, g, frames in rows:
        assert select.select_power(T, B, g).tolist() == frames


@pytest.mark.parametrize("T_max", [700])
def test_power_invariants(T_max):
    for T in range(0, T_max + 1):
        for B in (1, 2, 3, 5, 8, 17, 18, 19, 33, 64):
            s = select.select_power(T, B, 2.0)
            N = min(B, T)
            assert len(s) == N
            if N == 0:
                continue
            assert np.all(np.diff(s) > 0)
            assert s[-1] == T - 1
            assert s[0] >= 0
            if N >= 2:
                assert s[0] == 0
            if B >= T:
                assert s.tolist() == list(range(T))


def test_power_half_even_tie():
    # T=5, budget 3: d_1 = 1 + rint(2 * 0.25) = 1 + rint(0.5) = 1 (half to even)
    assert select.select_power(5, 3, 2.0).tolist() == [0, 3, 4]


def test_power_budget18_never_ties():
    """With budget 18, (T-18) * (i/17)**2 is never exactly k + 1/2, so the
    rounding mode of rint cannot matter for the preset's budget."""
    from fractions import Fraction
    for T in range(19, 3000):
        for i in range(18):
            frac = Fraction((T - 18) * i * i, 17 * 17)
            assert frac - (frac.numerator // frac.denominator) != Fraction(1, 2)


def test_recent_and_all():
    assert select.select_recent(10, 4).tolist() == [6, 7, 8, 9]
    assert select.select_recent(3, 4).tolist() == [0, 1, 2]
    assert select.select_all(4).tolist() == [0, 1, 2, 3]
    assert select.select_recent(0, 4).tolist() == []


def _anchor_recent_brute(T, F, R):
    n_seg = -(-T // F)
    return [f for f in range(T) if f % F == 0 or f // F >= n_seg - R]


def test_anchor_recent_brute_force():
    for T in range(0, 200):
        for F in (1, 3, 30):
            for R in (0, 1, 3):
                assert select.select_anchor_recent(T, F, R).tolist() == _anchor_recent_brute(T, F, R)


def test_anchor_recent_twelve_segments_keeps_99_frames():
    s = select.select_anchor_recent(360, 30, 3)
    assert len(s) == 99
    assert s[:9].tolist() == [0, 30, 60, 90, 120, 150, 180, 210, 240]
    assert s[9:].tolist() == list(range(270, 360))
