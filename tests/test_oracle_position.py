"""Pins of the oracle's query / KV normalisation and rotary positions
(oracle/position.py) against closed forms and the properties the pages state
("DeepSeek-V4" book ch. 2 "Normalization and position"; ch. 7 "Query and KV
normalization", "Partial rotary position embeddings", "Why the output is
de-rotated")."""

import math

import numpy as np

from oracle import position as P

FREQ = 10000.0 ** (-np.arange(32) * 2.0 / 64.0)


def test_rms_norm_closed_forms():
    # [3, 4]: mean square 12.5; with eps 0.5 the divisor is sqrt(13)
    y = P.rms_norm([3.0, 4.0], [1.0, 1.0], 0.5)
    assert np.allclose(y, [3 / math.sqrt(13), 4 / math.sqrt(13)], rtol=0, atol=1e-15)
    y = P.rms_norm([3.0, 4.0], [2.0, 3.0], 0.5)
    assert np.allclose(y, [6 / math.sqrt(13), 12 / math.sqrt(13)], rtol=0, atol=1e-15)
    # no mean subtraction: a constant vector stays (a layer norm would give 0)
    assert np.allclose(P.rms_norm(np.full(8, 2.5), np.ones(8), 0.0), np.ones(8))
    # unit mean square, scale invariance (eps = 0)
    x = np.random.default_rng(0).standard_normal((5, 512))
    y = P.rms_norm(x, np.ones(512), 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0)
    assert np.allclose(P.rms_norm(7.0 * x, np.ones(512), 0.0), y)
    # epsilon guards an all-zero vector
    assert np.all(P.rms_norm(np.zeros(4), np.ones(4), 1e-6) == 0.0)


def test_rope_rotates_pairs_of_the_last_coordinates():
    # one pair, frequency 1, angle pi/2: (1, 0) -> (0, 1), (0, 1) -> (-1, 0)
    y = P.rope([5.0, 1.0, 0.0], math.pi / 2, [1.0])
    assert np.allclose(y, [5.0, 0.0, 1.0], atol=1e-15)
    y = P.rope([0.0, 1.0], math.pi / 2, [1.0])
    assert np.allclose(y, [-1.0, 0.0], atol=1e-15)
    # two pairs with their own frequencies: angle pos * f_i on pair i
    y = P.rope([1.0, 0.0, 1.0, 0.0], 2.0, [0.5, 0.25])
    assert np.allclose(y, [math.cos(1.0), math.sin(1.0), math.cos(0.5), math.sin(0.5)], atol=1e-15)
    x = np.random.default_rng(1).standard_normal(512)
    y = P.rope(x, 12345, FREQ)
    assert np.array_equal(y[:448], x[:448])  # only the last 64 coordinates rotate
    assert np.isclose(np.linalg.norm(y), np.linalg.norm(x))
    assert np.array_equal(P.rope(x, 0, FREQ), x)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(512), rng.standard_normal(512)
    for t, s in ((1000, 3), (5, 77), (1 << 20, (1 << 20) - 129)):
        a = P.rope(q, t, FREQ) @ P.rope(k, s, FREQ)
        b = P.rope(q, t - s, FREQ) @ k
        assert np.isclose(a, b, rtol=1e-9, atol=1e-9)


def test_derotation_inverts_and_makes_the_output_relative():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(512)
    assert np.allclose(P.derotate(P.rope(x, 4321, FREQ), 4321, FREQ), x)
    # an output mixing the same stored vector at several source positions:
    # after de-rotation by the query position it depends only on the
    # positions relative to the query (shifting every position changes nothing)
    v = rng.standard_normal(512)
    p = rng.random(6)
    src = np.array([3, 10, 40, 41, 90, 100])

    def out(t, shift):
        o = sum(pj * P.rope(v, s + shift, FREQ) for pj, s in zip(p, src))
        return P.derotate(o, t + shift, FREQ)
    assert np.allclose(out(120, 0), out(120, 7777))
    assert not np.allclose(out(120, 0), out(121, 0))


def test_prepare_and_entry_position():
    rng = np.random.default_rng(4)
    x, g = rng.standard_normal(512), 1 + 0.1 * rng.standard_normal(512)
    y = P.prepare(x, g, 1e-6, 99, FREQ)
    assert np.allclose(y, P.rope(P.rms_norm(x, g, 1e-6), 99, FREQ))
    # normalisation commutes with the rotation when the scale is 1 on every
    # rotated pair (rotations keep the mean square)
    g1 = g.copy()
    g1[448:] = 1.0
    assert np.allclose(P.rms_norm(P.rope(x, 99, FREQ), g1, 1e-6), P.prepare(x, g1, 1e-6, 99, FREQ))
    assert P.entry_position(3, 4) == 12 and P.entry_position(0, 128) == 0
