"""CPU checks of the parity rules in tests/compare.py (no GPU): the e4m3
rounding alternatives of a produced key and the bound-aware top-k check."""

import numpy as np

from tests.compare import e4m3_alternatives, score_bounds, topk_check, topk_check_bounds


def test_e4m3_alternatives_only_near_a_rounding_boundary():
    # scale = 448 / 448 = 1: y = x.  1.0625 is the midpoint of the e4m3
    # values 1.0 and 1.125; 1.03 is not near any midpoint
    alts = e4m3_alternatives(np.array([448.0, 1.0625, -1.03]))
    vals = sorted(a[1] for a in alts)
    assert len(alts) == 2 and vals == [1.0, 1.125]
    assert all(a[0] == 448.0 and a[2] == -1.0 for a in alts)
    assert len(e4m3_alternatives(np.array([448.0, 1.0625 * (1 + 1e-4), 3.0]))) == 1
    # two ambiguous coordinates: four rows
    assert len(e4m3_alternatives(np.array([448.0, 1.0625, -2.125]))) == 4


def test_topk_check_bounds_accepts_only_swaps_the_bounds_allow():
    scores = np.array([5.0, 4.0, 3.0, 2.9, 1.0])
    k = 3
    oracle = np.array([0, 1, 2])
    swapped = np.array([0, 1, 3, -1])
    assert not topk_check(swapped, 3, oracle, scores, k)[0]
    # entry 3 may score up to 3.1 and entry 2 down to 2.8 under another rounding
    q = np.array([[1.0]])
    w = np.array([1.0])
    amb = {3: [np.array([2.9]), np.array([3.1])], 2: [np.array([3.0]), np.array([2.8])]}
    bd = score_bounds(q, w, amb)
    assert bd == {3: (2.9, 3.1), 2: (2.8, 3.0)}
    assert topk_check_bounds(swapped, 3, oracle, scores, k, bd)[0]
    # bounds on an unrelated entry do not excuse the swap
    assert not topk_check_bounds(swapped, 3, oracle, scores, k, {4: (0.5, 1.5)})[0]
    # nor bounds too narrow to reach
    assert not topk_check_bounds(swapped, 3, oracle, scores, k, {3: (2.9, 2.95)})[0]
