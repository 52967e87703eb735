"""Pins for the oracle's arithmetic, each tied to something other than the
oracle itself: the pages' worked examples (tests/golden), closed forms,
special cases that reduce to a library routine, and brute force on tiny
inputs.  Each test names the plausible mistakes it would catch."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import csa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# compressor
# ---------------------------------------------------------------------------

def test_compressor_worked_example_9_6():
    """Book ch. 5 scalar example; catches a wrong branch/block assignment
    (8.0, 8.8, 11.6) and softmax over coordinates instead of positions."""
    g = golden("compressor_scalar_example.json")
    ca = np.array(g["content_a"])[:, None]
    za = np.array(g["logits_a"])[:, None]
    cb = np.array(g["content_b_prev"])[:, None]
    zb = np.array(g["logits_b_prev"])[:, None]
    out = csa.compress_entry(ca, za, None, cb, zb, None)
    assert out.shape == (1,)
    assert abs(out[0] - g["expected"]) < 1e-12
    # the same through the chunk API: previous block supplied as state
    out2 = csa.compress(ca, za, g["m"], None, np.zeros_like(ca), np.zeros_like(za), None, cb, zb)
    assert abs(out2[0, 0] - g["expected"]) < 1e-12


def test_compressor_uniform_logits_give_block_mean():
    """Closed form: equal logits -> block mean (HCA form); catches dropped or
    misplaced source positions and a softmax over the wrong axis."""
    rng = np.random.default_rng(0)
    m, c, T = 8, 5, 32
    C = rng.standard_normal((T, c))
    Z = np.full((T, c), 0.37)
    out = csa.compress(C, Z, m)
    assert np.allclose(out, C.reshape(T // m, m, c).mean(axis=1), rtol=0, atol=1e-13)


def test_compressor_overlap_uniform_closed_form_and_start_rule():
    """Overlap with equal logits: entry i = (sum of block i via a + sum of
    block i-1 via b) / 2m; entry 0 (no previous block) = mean of block 0 via a
    (book ch. 5 start-of-sequence rule).  Catches b taken from the wrong block
    and a missing -inf for the absent branch."""
    rng = np.random.default_rng(1)
    m, c, T = 4, 6, 24
    Ca, Cb = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    Z = np.zeros((T, c))
    out = csa.compress(Ca, Z, m, None, Cb, Z, None)
    A = Ca.reshape(-1, m, c).sum(1)
    Bs = Cb.reshape(-1, m, c).sum(1)
    assert np.allclose(out[0], A[0] / m, atol=1e-13)
    for i in range(1, T // m):
        assert np.allclose(out[i], (A[i] + Bs[i - 1]) / (2 * m), atol=1e-13)


def test_compressor_bias_sets_the_weights():
    """Closed form: Z = 0 and B[j, r] = log p[j, r] give sum_j p[j, r] C[j, r]
    per coordinate.  Catches a dropped bias, bias indexed [c][m], and one
    weight per token instead of one per coordinate."""
    rng = np.random.default_rng(2)
    m, c = 4, 3
    p = rng.random((m, c)) + 0.1
    p /= p.sum(axis=0, keepdims=True)
    C = rng.standard_normal((m, c))
    out = csa.compress_entry(C, np.zeros((m, c)), np.log(p))
    assert np.allclose(out, (p * C).sum(axis=0), atol=1e-13)
    # the overlap branch's own bias
    pb = rng.random((2 * m, c)) + 0.1
    pb /= pb.sum(axis=0, keepdims=True)
    Cb = rng.standard_normal((m, c))
    out = csa.compress_entry(C, np.zeros((m, c)), np.log(pb[:m]), Cb, np.zeros((m, c)),
                             np.log(pb[m:]))
    assert np.allclose(out, (pb[:m] * C).sum(0) + (pb[m:] * Cb).sum(0), atol=1e-13)


def test_compressor_invariants():
    """Shift invariance per coordinate, and the result stays inside the
    per-coordinate hull of its sources (weights are a distribution)."""
    rng = np.random.default_rng(3)
    m, c = 4, 16
    Ca, Cb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    Za, Zb = rng.standard_normal((m, c)) * 3, rng.standard_normal((m, c)) * 3
    Ba, Bb = rng.standard_normal((m, c)), rng.standard_normal((m, c))
    base = csa.compress_entry(Ca, Za, Ba, Cb, Zb, Bb)
    shift = rng.standard_normal(c) * 50
    shifted = csa.compress_entry(Ca, Za + shift, Ba, Cb, Zb + shift, Bb)
    assert np.allclose(base, shifted, atol=1e-12)
    allC = np.concatenate([Ca, Cb])
    assert np.all(base <= allC.max(0) + 1e-12) and np.all(base >= allC.min(0) - 1e-12)


def test_scalar_logit_form_weights_per_token():
    """One logit per token shared by all coordinates: with x whose first
    coordinate dominates w.x, the entry tends to the max-logit token."""
    m, c = 4, 3
    x = np.zeros((m, c))
    x[:, 1] = [1, 2, 3, 4]
    x[2, 0] = 100.0  # w = e_0 gives token 2 a logit of 100
    w = np.array([1.0, 0, 0])
    out = csa.compress(x, csa.scalar_logits(x, w), m)
    assert np.allclose(out[0], x[2], atol=1e-30)


def test_entry_counts_from_pages():
    g = golden("entry_counts.json")
    for case in g["cases"]:
        assert csa.entry_count(case["n"], case["m"]) == (case["entries"], case["tail"])


def test_visibility_and_window_cover_every_past_position():
    """Under the default reading, any position <= t lies in a visible entry
    or in the window whenever n_win >= m, and no visible entry contains a
    position > t (causality of the compressed path)."""
    for m in (1, 4, 128):
        for n_win in (m, 128):
            for t in list(range(0, 600)) + [10 ** 6 + 3]:
                nv = csa.visible_entries(t, m, 10 ** 9)
                assert nv * m - 1 <= t  # last visible entry ends at or before t
                covered_hi = nv * m  # entries cover [0, nv*m)
                wlo = csa.window_positions(t, n_win)[0]
                assert wlo <= covered_hi  # no gap between entries and window
    assert csa.visible_entries(7, 4, 10) == 1
    assert csa.visible_entries(7, 4, 10, csa.VIS_COMPLETED) == 2
    assert csa.visible_entries(100, 4, 3) == 3


# ---------------------------------------------------------------------------
# indexer and top-k
# ---------------------------------------------------------------------------

def test_indexer_hand_example():
    g = golden("indexer_hand_example.json")
    s = csa.index_scores(g["q"], g["w"], g["keys"])
    assert np.allclose(s, g["expected_scores"], atol=1e-14)
    assert list(csa.topk_select(s, g["k"])) == g["expected_topk"]


def test_indexer_single_head_is_relu_dot():
    """H_I = 1, w = 1: the score is max(0, q.k) from numpy's dot."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 16))
    K = rng.standard_normal((50, 16))
    s = csa.index_scores(q, [1.0], K)
    ref = np.array([max(0.0, float(np.dot(q[0], k))) for k in K])
    assert np.allclose(s, ref, atol=1e-13)
    assert (s == 0).any() and (s > 0).any()


def test_indexer_linearity_and_homogeneity():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((6, 8))
    K = rng.standard_normal((40, 8))
    w1, w2 = rng.standard_normal(6), rng.standard_normal(6)
    s = lambda w, KK=K: csa.index_scores(q, w, KK)  # noqa: E731
    assert np.allclose(s(w1 + w2), s(w1) + s(w2), atol=1e-12)
    assert np.allclose(s(w1, 2.5 * K), 2.5 * s(w1), atol=1e-12)
    assert np.all(s(np.abs(w1)) >= 0)
    # negative weights can make scores negative (no positivity constraint)
    assert np.any(s(-np.abs(w1)) < 0)


def test_topk_brute_force_with_ties():
    """Entry s is selected iff fewer than k entries beat it, where t beats s
    when I_t > I_s or (I_t == I_s and t < s); compared with the oracle and
    with torch.topk's value set."""
    rng = np.random.default_rng(6)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 45))
        scores = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
        want = [s for s in range(n)
                if sum((scores[t] > scores[s]) or (scores[t] == scores[s] and t < s)
                       for t in range(n)) < k]
        got = csa.topk_select(scores, k)
        assert list(got) == want
        vals = torch.topk(torch.from_numpy(scores), min(k, n)).values.numpy()
        assert np.array_equal(np.sort(scores[got]), np.sort(vals))


def test_topk_keeps_all_when_fewer_than_k():
    s = np.array([3.0, -1.0, 2.0])
    assert list(csa.topk_select(s, 8)) == [0, 1, 2]
    assert list(csa.topk_select(np.zeros(0), 4)) == []


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _sdpa_causal_mqa(q_all, x, scale):
    """Textbook causal MQA attention from torch's SDPA (float64, CPU)."""
    T, H, c = q_all.shape
    qt = torch.from_numpy(q_all).permute(1, 0, 2)[None]  # [1][H][T][c]
    kt = torch.from_numpy(x)[None, None].expand(1, H, T, c)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_csa_with_m1_full_budget_is_full_causal_attention():
    """m = 1, k >= n, window of 1, no sink: CSA reduces to exact causal
    softmax attention over positions 0..t (every token is its own entry,
    visible entries are 0..t-1 and the window adds t)."""
    from oracle.formats import Stored
    rng = np.random.default_rng(7)
    T, H, c, d_I, H_I = 24, 3, 8, 4, 2
    x = rng.standard_normal((T, c)).astype(np.float32)
    q = rng.standard_normal((T, H, c))
    ref = _sdpa_causal_mqa(q, x.astype(np.float64), 1 / math.sqrt(c))
    kv = Stored(x, "f32")
    keys = Stored(rng.standard_normal((T, d_I)).astype(np.float32), "f32")
    for t in range(T):
        o, lse, sel, _ = csa.csa_query(q[t], rng.standard_normal((H_I, d_I)),
                                       rng.standard_normal(H_I), t, kv, keys, T,
                                       lambda p: x[p].astype(np.float64), None,
                                       m=1, k=T, n_win=1, scale=1 / math.sqrt(c))
        assert list(sel) == list(range(t))
        assert np.allclose(o, ref[t], atol=1e-12, rtol=0)


def test_sink_worked_example_0_4():
    g = golden("sink_example.json")
    # one real row of value 1 with logit log(4) and a sink logit log(6)
    q = np.array([[math.log(g["real_mass"])]])
    rows = np.array([[1.0]])
    o, lse = csa.attend(q, rows, sink=np.array([math.log(g["sink_mass"])]), scale=1.0)
    assert abs(o[0, 0] - g["expected_real_weight_sum"]) < 1e-14
    assert abs(lse[0] - math.log(g["real_mass"] + g["sink_mass"])) < 1e-14


def test_sink_closed_form_and_sink_only_head():
    rng = np.random.default_rng(8)
    H, R, c = 4, 30, 16
    q = rng.standard_normal((H, c))
    rows = rng.standard_normal((R, c))
    o0, lse0 = csa.attend(q, rows, None, 0.25)
    z = rng.standard_normal(H)
    o1, lse1 = csa.attend(q, rows, z, 0.25)
    L = np.exp(lse0)
    assert np.allclose(o1, o0 * (L / (L + np.exp(z)))[:, None], atol=1e-12)
    assert np.allclose(lse1, np.log(L + np.exp(z)), atol=1e-12)
    logits = 0.25 * q @ rows.T
    zs = logits.max(axis=1) + 40
    o2, _ = csa.attend(q, rows, zs, 0.25)
    assert np.abs(o2).max() <= 1e-6 * np.abs(rows).max()


def test_split_merge_invariance():
    rng = np.random.default_rng(9)
    H, R, c = 5, 57, 12
    q = rng.standard_normal((H, c))
    rows = rng.standard_normal((R, c)) * 3
    z = rng.standard_normal(H)
    o, lse = csa.attend(q, rows, z, 0.3)
    cuts = [0, 7, 8, 30, 57]
    parts = [csa.attend_partial(q, rows[a:b], 0.3) for a, b in zip(cuts, cuts[1:])]
    o2, lse2 = csa.merge_partials(parts, z)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)


def test_csa_with_budget_covering_all_entries_equals_hca():
    from oracle.formats import Stored
    rng = np.random.default_rng(10)
    E, c, H, d_I, H_I, m = 40, 8, 3, 4, 2, 4
    kv = Stored(rng.standard_normal((E, c)).astype(np.float32), "f32")
    keys = Stored(rng.standard_normal((E, d_I)).astype(np.float32), "f32")
    win = rng.standard_normal((200, c))
    t = 150
    q = rng.standard_normal((H, c))
    z = rng.standard_normal(H)
    o1, l1, sel, _ = csa.csa_query(q, rng.standard_normal((H_I, d_I)), rng.standard_normal(H_I),
                                   t, kv, keys, E, lambda p: win[p], z, m, 64, 16, 0.3)
    o2, l2 = csa.hca_query(q, t, kv, E, lambda p: win[p], z, m, 16, 0.3)
    assert len(sel) == 37  # floor(150/4)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(l1, l2, atol=1e-12)


def test_e4m3_quantizer_matches_torch_cast():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 128)) * np.abs(rng.standard_t(3, size=(64, 1)))).astype(
        np.float32)
    vals, scale = csa.e4m3_quantize_rows(x.astype(np.float64))
    assert scale.dtype == np.float32
    y = np.clip(x.astype(np.float64) / scale.astype(np.float64)[:, None], -448, 448)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(vals, ref * scale.astype(np.float64)[:, None])


@pytest.mark.parametrize("vis", [csa.VIS_PRIOR_BLOCKS, csa.VIS_COMPLETED])
def test_causality_of_prefill_queries(vis):
    """Perturbing every input at positions > t leaves query t unchanged
    (book ch. 5: the same causal rule applies to selection scores)."""
    import workloads
    from oracle import layer
    a, _ = workloads.flash_prefill(seed=11, T=32, n0=64, H=2, c=16, H_I=2, d_I=8, k=4)
    a["vis"] = vis
    kv_new, idx_new = layer.prefill_entries(a, 0)
    t_i = 13
    ref = layer.prefill_query(a, 0, t_i, kv_new, idx_new)
    b = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in a.items()}
    rng = np.random.default_rng(0)
    for name in ("ca", "za", "cb", "zb", "ica", "iza", "icb", "izb", "q", "q_idx", "w_idx"):
        arr = b[name]
        arr[0, t_i + 1:] = rng.permutation(arr[0, t_i + 1:].reshape(-1)).reshape(
            arr[0, t_i + 1:].shape)
    wlo = t_i + 1 + (a["n_win"] - 1)
    b["win"][0, wlo:] = rng.permutation(b["win"][0, wlo:].reshape(-1)).reshape(
        b["win"][0, wlo:].shape)
    kv2, idx2 = layer.prefill_entries(b, 0)
    got = layer.prefill_query(b, 0, t_i, kv2, idx2)
    assert np.array_equal(ref["o"], got["o"]) and np.array_equal(ref["sel"], got["sel"])
