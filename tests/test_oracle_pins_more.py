"""More pins for the oracle, each against something other than the oracle's
own formula: hand-computed values, a textbook routine written out with plain
loops, and brute force on tiny inputs.  Each test names the mistakes it
catches."""

import math

import numpy as np

import workloads
from oracle import csa, layer
from oracle.formats import Stored, f64_to_bf16_bits


# ---------------------------------------------------------------------------
# indexer over a stored cache, across the decode chunk boundary
# ---------------------------------------------------------------------------

def _loop_scores(q, w, K):
    """I[s] = sum_h w[h] max(0, sum_d q[h,d] K[s,d]) with Python loops."""
    out = []
    for s in range(K.shape[0]):
        tot = 0.0
        for h in range(q.shape[0]):
            dot = 0.0
            for d in range(q.shape[1]):
                dot += float(q[h, d]) * float(K[s, d])
            tot += float(w[h]) * max(0.0, dot)
        out.append(tot)
    return np.array(out)


def test_index_scores_stored_across_chunk_boundaries():
    """The stored-cache scorer decodes the cache chunk by chunk; a dropped,
    repeated or shifted chunk, or a wrong last-chunk bound, changes some
    score.  Checked against Python loops on a small chunk size (many
    boundaries, a ragged last chunk), and at the default 65,536-row chunk on
    70,001 rows (one boundary, a ragged tail) against the one-shot scorer on
    the whole decoded array."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 4))
    w = rng.standard_normal(3)
    K = Stored(f64_to_bf16_bits(rng.standard_normal((23, 4))), "bf16")
    ref = _loop_scores(q, w, K.all())
    for n, chunk in ((23, 5), (20, 7), (1, 5), (0, 5)):
        got = csa.index_scores_stored(q, w, K, n, chunk=chunk)
        assert got.shape == (n,)
        assert np.allclose(got, ref[:n], rtol=0, atol=1e-12)
    big = Stored(f64_to_bf16_bits(rng.standard_normal((70001, 4))), "bf16")
    full = csa.index_scores(q, w, big.all())
    for n in (65535, 65536, 65537, 70001):
        got = csa.index_scores_stored(q, w, big, n)
        assert np.array_equal(got, full[:n])
    # rows straddling the boundary, by the loops
    i = np.arange(65530, 65542)
    assert np.allclose(csa.index_scores_stored(q, w, big, 70001)[i], _loop_scores(q, w, big.rows(i)),
                       rtol=0, atol=1e-12)


def test_csa_query_budget_below_visible_is_brute_force():
    """k smaller than the visible count: the selected set is the k best by
    (score descending, id ascending) computed by plain sorting of loop
    scores, and the output is the attention over exactly those entries and the
    window rows of positions t-n_win+1 .. t (attention written out with
    loops).  Catches selecting from the wrong end, visibility off by one,
    window rows from the wrong positions, and a dropped sink."""
    rng = np.random.default_rng(12)
    m, n_ent, c, H, d_I, H_I, k, n_win = 4, 40, 6, 2, 5, 3, 7, 5
    t = 4 * 37 + 2  # visible: floor(t/m) = 37 of the 40 cached entries
    kv = Stored(rng.standard_normal((n_ent, c)).astype(np.float32), "f32")
    keys = Stored(rng.standard_normal((n_ent, d_I)).astype(np.float32), "f32")
    q = rng.standard_normal((H, c))
    qi = rng.standard_normal((H_I, d_I))
    w = np.abs(rng.standard_normal(H_I))
    # an exact tie at the boundary: the (k+1)-th best entry takes the k-th
    # best's key, and the lower of the two ids must win
    pre = _loop_scores(qi, w, keys.all()[:37])
    order = sorted(range(37), key=lambda s: (-pre[s], s))
    keys.data[order[k]] = keys.data[order[k - 1]]
    tie = sorted((order[k - 1], order[k]))
    sink = rng.standard_normal(H)
    raw = rng.standard_normal((t + 1, c))
    scale = 0.4
    o, lse, sel, scores = csa.csa_query(q, qi, w, t, kv, keys, n_ent, lambda p: raw[np.asarray(p)],
                                        sink, m, k, n_win, scale)
    ls = _loop_scores(qi, w, keys.all()[:37])
    assert np.allclose(scores, ls, atol=1e-12) and len(scores) == 37
    best = sorted(range(37), key=lambda s: (-ls[s], s))[:k]
    assert list(sel) == sorted(best)
    assert tie[0] in best and tie[1] not in best
    rows = [kv.all()[s] for s in sorted(best)] + [raw[p] for p in range(t - n_win + 1, t + 1)]
    for h in range(H):
        lg = [scale * sum(q[h, d] * r[d] for d in range(c)) for r in rows]
        M = max(lg + [sink[h]])
        ex = [math.exp(x - M) for x in lg]
        den = sum(ex) + math.exp(sink[h] - M)
        ref = [sum(e * r[d] for e, r in zip(ex, rows)) / den for d in range(c)]
        assert np.allclose(o[h], ref, atol=1e-12)
        assert abs(lse[h] - (M + math.log(den))) < 1e-12


# ---------------------------------------------------------------------------
# the tiny whole-context case: entries and per-query wiring
# ---------------------------------------------------------------------------

def _textbook_causal(q, xs, scale):
    """softmax(scale q . x_j) over j, weighted sum of x_j, with loops."""
    H, c = q.shape
    out = np.zeros((H, c))
    for h in range(H):
        lg = [scale * sum(q[h, d] * x[d] for d in range(c)) for x in xs]
        M = max(lg)
        ex = [math.exp(v - M) for v in lg]
        den = sum(ex)
        for d in range(c):
            out[h, d] = sum(e * x[d] for e, x in zip(ex, xs)) / den
    return out


def test_tiny_query_reduces_to_causal_attention():
    """With m = 1 (an entry is its one token whatever its logit), a budget
    covering every entry, a window of one and no sink, every tiny query is
    plain causal softmax attention over x[0 .. t].  Catches window rows read
    from the indexer's raw keys or from the wrong positions, the query's own
    token missing or doubled, and entries compressed from the wrong stream."""
    g = workloads.tiny_case(seed=5, n=48, c=6, H=2, H_I=2, d_I=3, k=64, Tq=4, m=1, n_win=1)
    g["sink"] = np.full(g["H"], -np.inf)
    g["q_pos"] = np.array([[0, 7, 30, 47]], dtype=np.int64)
    kv, keys = layer.tiny_entries(g)
    x = g["x"][0].astype(np.float64)
    assert np.array_equal(kv, x) and np.array_equal(keys, g["x_idx"][0].astype(np.float64))
    for i in range(4):
        t = int(g["q_pos"][0][i])
        o, _, sel, _ = layer.tiny_query(g, i, kv, keys)
        assert list(sel) == list(range(t))
        ref = _textbook_causal(g["q"][0][i].astype(np.float64), [x[j] for j in range(t + 1)], g["scale"])
        assert np.allclose(o, ref, atol=1e-12)


def test_tiny_entries_zero_logit_weights_give_block_means():
    """w = 0 makes every token's scalar logit 0: each entry is the plain mean
    of its m tokens, for the main entries and the indexer keys alike.  Catches
    blocks of the wrong length or offset and the two streams swapped."""
    g = workloads.tiny_case(seed=6, n=64, c=5, H=2, H_I=2, d_I=3, k=8, Tq=2, m=4, n_win=8)
    g["w_cmp"] = np.zeros_like(g["w_cmp"])
    g["w_cmp_idx"] = np.zeros_like(g["w_cmp_idx"])
    kv, keys = layer.tiny_entries(g)
    x, xi = g["x"][0].astype(np.float64), g["x_idx"][0].astype(np.float64)
    for i in range(16):
        for r in range(5):
            assert abs(kv[i, r] - np.float32(sum(x[4 * i + j, r] for j in range(4)) / 4)) < 1e-6
        for r in range(3):
            assert abs(keys[i, r] - np.float32(sum(xi[4 * i + j, r] for j in range(4)) / 4)) < 1e-6


def test_scalar_logits_are_dot_products():
    """Hand-computed: x = [[2, 0], [0, 2]], w = [ln 3, 0] give logits
    2 ln 3 and 0, weights 9/10 and 1/10, entry (1.8, 0.2).  A sum of x
    instead of w . x would give equal weights (1, 1); x . w transposed or
    w ignored would give other values."""
    x = np.array([[2.0, 0.0], [0.0, 2.0]])
    w = np.array([math.log(3.0), 0.0])
    lg = csa.scalar_logits(x, w)
    assert lg.shape == (2, 1)
    assert abs(lg[0, 0] - 2 * math.log(3.0)) < 1e-15 and lg[1, 0] == 0.0
    out = csa.compress(x, lg, 2)
    assert np.allclose(out[0], [1.8, 0.2], atol=1e-15)
