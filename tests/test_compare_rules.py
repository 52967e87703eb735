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


def test_mxfp4_alternatives_element_and_scale_boundaries():
    from oracle.formats import mxfp4_quantize
    from tests.compare import mxfp4_alternatives
    # block max 6 -> scale 2^(2 - 2) = 1: y = x.  0.75 is the midpoint of
    # 0.5 and 1.0 (E2M1 codes 1 and 2); 1.1 is near no midpoint
    x = np.zeros(32)
    x[0], x[1], x[2] = 6.0, 0.75, -1.1
    alts = mxfp4_alternatives(x)
    assert len(alts) == 2
    assert sorted(a[1] for a in alts) == [0.5, 1.0]
    assert all(a[0] == 6.0 and a[2] == -1.0 for a in alts)
    assert any(np.array_equal(a, mxfp4_quantize(x)[2]) for a in alts)
    x[1] = 0.7
    assert len(mxfp4_alternatives(x)) == 1
    # block max exactly 4 = 2^2: a float32 maximum a hair below selects the
    # scale 2^-1 (elements / 0.5: 4 -> 8 saturates to 6), exactly 4 the
    # scale 1; the second block is unambiguous
    y = np.zeros(64)
    y[0], y[1], y[33] = 4.0, 1.3, 2.2
    alts = mxfp4_alternatives(y)
    assert len(alts) == 2
    assert sorted(a[0] for a in alts) == [3.0, 4.0]
    assert all(a[33] == 2.0 for a in alts)


def test_topk_check_intervals_tie_rule_and_uncertainty():
    from tests.compare import bf16_score_intervals, topk_check_intervals
    lo = np.array([1.0, 2.0, 2.0, 3.0, 2.0])
    hi = lo.copy()
    k = 3
    # certain scores: {3} plus the two lowest-id entries at 2.0
    assert topk_check_intervals([1, 2, 3], 3, k, lo, hi)[0]
    ok, _, msg = topk_check_intervals([1, 3, 4], 3, k, lo, hi)
    assert not ok and "tie" in msg
    assert not topk_check_intervals([0, 1, 3], 3, k, lo, hi)[0]
    assert not topk_check_intervals([1, 2], 2, k, lo, hi)[0]
    # entry 4 may round up to 2.015625 (one bf16 step above 2): then it may
    # replace entry 2
    hi2 = hi.copy()
    hi2[4] = 2.015625
    ok, unc, _ = topk_check_intervals([1, 3, 4], 3, k, lo, hi2)
    assert ok and unc == 1
    # intervals from exact scores and error bounds: 2 + 1e-9 rounds to 2,
    # and with an error bound reaching the midpoints on both sides (bf16
    # spacing 2^-6 above 2, 2^-7 below) either neighbour is possible
    s = np.array([2.0 + 1e-9, 1.0])
    lo3, hi3 = bf16_score_intervals(s, np.array([1e-12, 0.0]))
    assert lo3[0] == hi3[0] == 2.0
    lo4, hi4 = bf16_score_intervals(s, np.array([0.0079, 0.0]))
    assert lo4[0] == 1.9921875 and hi4[0] == 2.015625
