"""Parity rules between the HIP path and the oracle.

* Top-k sets are bit-exact, except that an id in the symmetric difference is
  allowed when its oracle (float64) score lies within 1e-6 relative of the
  oracle's k-th score tau (the float32 score-gap rule), or within the float32
  evaluation error bound of the two scores when that is larger (signed head
  weights make the score a sum with cancellation: score_error_bound).  Such
  swaps are counted and reported.
* Layer-produced e4m3 keys: a stored code may be either neighbour when the
  value sits within float32 accuracy of a rounding boundary; selections are
  accepted when some such rounding makes them a top-k (topk_check_bounds).
* MXFP4 keys the layer produces: a block's scale or an element's code may
  take either rounding when the value sits within float32 accuracy of a
  boundary (mxfp4_alternatives).
* bf16 index scores: each entry's score is known within the bf16 roundings
  of its float32 error interval; the selection must be the exact top-k,
  ties to the lower id, of some scores within those intervals
  (topk_check_intervals).
* Floating outputs: per row, max|gpu - ref| / max(max|ref|, 1e-3 * median
  row max) <= tol, with tol = 1e-4 for float32 paths and 2e-2 for bfloat16.
  The worst row, the global max-abs error and the lse error are reported.
"""

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def score_error_bound(q, w, K):
    """Worst-case |float32 score - exact score| of every row of K: the score
    is a sum over d_I exact products per head (one float32 sum each), a
    product by the head weight (and scales), a sum over H_I heads and a
    product by the key scale, so a float32 evaluation in any order is within
    (d_I + H_I + 3) u M_s of the exact score (the standard bound for
    floating-point sums), u = 2**-24, M_s the same score of |q|, |w| and |K|
    (no cancellation)."""
    from oracle.csa import index_scores
    q = np.abs(np.asarray(q, np.float64))
    H_I, d_I = q.shape
    M = index_scores(q, np.abs(np.asarray(w, np.float64)), np.abs(np.asarray(K, np.float64)))
    return (d_I + H_I + 3) * 2.0 ** -24 * M


def topk_check(gpu_ids, gpu_cnt, oracle_sel, scores, k, rel_gap=1e-6, err=None):
    """Returns (ok, n_swaps, message).  ``err`` (optional): an array of
    per-entry float32 evaluation error bounds (score_error_bound), or a
    function returning it, evaluated only when the sets differ; an id in
    the symmetric difference is then also allowed when its score lies within
    its bound plus the k-th entry's bound of tau."""
    gpu = np.asarray(gpu_ids)[:int(gpu_cnt)]
    if np.any(np.diff(gpu) <= 0):
        return False, 0, "gpu ids not strictly ascending"
    if len(gpu) != len(oracle_sel):
        return False, 0, f"count {len(gpu)} != oracle {len(oracle_sel)}"
    if np.array_equal(gpu, oracle_sel):
        return True, 0, ""
    diff = np.setxor1d(gpu, oracle_sel)
    if diff.size and (diff.min() < 0 or diff.max() >= len(scores)):
        return False, 0, "gpu id outside the visible range"
    order = np.lexsort((np.arange(len(scores)), -np.asarray(scores)))
    kth = order[min(k, len(scores)) - 1]
    tau = scores[kth]
    tol = np.full(len(diff), rel_gap * abs(tau))
    e = None
    if err is not None:
        e = np.asarray(err() if callable(err) else err, np.float64)
        tol = np.maximum(tol, e[diff] + e[kth])
    bad = [int(s) for s, t in zip(diff, tol) if abs(scores[s] - tau) > t]
    if bad:
        extra = "" if e is None else f", fp32 error bound at tau {e[kth]:.3g}"
        return False, len(diff), f"ids {bad[:8]} differ with score gaps beyond {rel_gap}{extra} (tau={tau})"
    return True, len(diff) // 2, ""


# relative accuracy of a float32 fold's value (softmax of a few logits,
# hardware exp, accumulation, the division by the scale)
FOLD_REL = 4e-6


def e4m3_alternatives(raw_row, rel=FOLD_REL, max_amb=6):
    """Every value row (codes times scale, float64) that rounding ``raw_row``
    to e4m3 with one scale per row may give when the value is computed in
    float32: the oracle's rounding, plus the other neighbouring code for each
    coordinate whose value / scale lies within ``rel`` of a rounding boundary
    (both roundings are then correct within the float32 computation).  At
    most 2**max_amb rows."""
    from oracle.csa import e4m3_quantize_rows
    x = np.asarray(raw_row, np.float64)
    base, scale = e4m3_quantize_rows(x[None])
    base, sc = base[0], float(scale[0])
    y = np.abs(x) / sc
    _, e = np.frexp(np.where(y > 0, y, 1.0))
    sp = np.ldexp(1.0, np.maximum(e - 4, -9))
    frac = y / sp - np.floor(y / sp)
    amb = np.where((np.abs(frac - 0.5) * sp <= rel * np.maximum(y, 1e-30)) & (y < 448.0))[0]
    assert len(amb) <= max_amb, f"{len(amb)} ambiguous codes in one key"
    rows = [base]
    for i in amb:
        lo, hi = np.floor(y[i] / sp[i]) * sp[i], np.ceil(y[i] / sp[i]) * sp[i]
        other = hi if abs(base[i]) / sc == lo else lo
        alt = []
        for r in rows:
            r2 = r.copy()
            r2[i] = np.copysign(other * sc, x[i])
            alt.append(r2)
        rows += alt
    return rows


def ambiguous_e4m3_keys(raw_rows, ids, rel=FOLD_REL):
    """{id: alternative value rows} for the layer-produced e4m3 keys (given
    before rounding) whose stored codes are not settled by float32 accuracy;
    keys with a single valid rounding are left out."""
    out = {}
    for s, raw in zip(ids, raw_rows):
        alts = e4m3_alternatives(raw, rel)
        if len(alts) > 1:
            out[int(s)] = alts
    return out


def score_bounds(q, w, amb):
    """{id: (lo, hi)} index scores of each ambiguous key's alternatives, for
    one query (q [H_I][d_I], w [H_I], as the oracle scores them)."""
    from oracle.csa import index_scores
    out = {}
    for s, alts in amb.items():
        sc = index_scores(q, w, np.array(alts))
        out[s] = (float(sc.min()), float(sc.max()))
    return out


def topk_check_bounds(gpu_ids, gpu_cnt, oracle_sel, scores, k, bounds, rel_gap=1e-6, err=None):
    """topk_check for selections over keys some of whose scores are only
    known within bounds ({id: (lo, hi)}, see score_bounds): the GPU set S
    is accepted when some scores within the bounds make it a top-k, i.e.
    min over S of the upper bounds >= max over the rest of the lower bounds,
    up to the float32 score-gap rule.  Returns (ok, n_swaps, message)."""
    ok, swaps, msg = topk_check(gpu_ids, gpu_cnt, oracle_sel, scores, k, rel_gap, err)
    if ok or not bounds:
        return ok, swaps, msg
    gpu = np.asarray(gpu_ids)[:int(gpu_cnt)]
    if len(gpu) != len(oracle_sel) or np.any(np.diff(gpu) <= 0) or gpu.min() < 0 or gpu.max() >= len(scores):
        return ok, swaps, msg
    lo = np.array(scores, np.float64)
    hi = lo.copy()
    for s, (a, b) in bounds.items():
        if s < len(lo):
            lo[s], hi[s] = a, b
    inside = np.zeros(len(lo), bool)
    inside[gpu] = True
    tau = np.sort(scores)[::-1][min(k, len(scores)) - 1]
    if inside.all() or hi[inside].min() >= lo[~inside].max() - rel_gap * abs(tau):
        return True, len(np.setxor1d(gpu, oracle_sel)) // 2, ""
    return False, 0, msg + " (also beyond the e4m3 rounding bounds)"


def decode_err(g, b, ref):
    """score_error_bound of the entries visible to sequence b of decode
    workload g (the cache rows, then the key the step folded), as a
    function for topk_check's lazy ``err``."""
    def f():
        from oracle.formats import Stored
        from oracle.layer import CacheView
        idk = g["idx_dtype"]
        sc = g.get("idx_scale")
        keys = CacheView(Stored(g["idx_cache"][b], idk, None if sc is None else sc[b]), int(g["n_entries"][b]),
                         np.array(ref["folded_idx"]) if ref["folded_idx"] else None)
        qs = g.get("q_scale")
        q = Stored(g["q_idx"][b], idk, None if qs is None else qs[b]).all()
        return score_error_bound(q, g["w_idx"][b], keys.rows(slice(0, len(ref["scores"]))))
    return f


def prefill_err(g, b, i, idx_new, n_vis):
    """score_error_bound for chunk query i of sequence b of prefill workload
    g over its n_vis visible entries (cache rows, then the chunk's keys)."""
    def f():
        from oracle.formats import Stored
        from oracle.layer import CacheView
        idk = g["idx_dtype"]
        sc = g.get("idx_scale")
        keys = CacheView(Stored(g["idx_cache"][b], idk, None if sc is None else sc[b]), int(g["n_entries"][b]),
                         idx_new)
        qs = g.get("q_scale")
        q = Stored(g["q_idx"][b][i], idk, None if qs is None else qs[b][i]).all()
        return score_error_bound(q, g["w_idx"][b][i], keys.rows(slice(0, n_vis)))
    return f


def mxfp4_alternatives(raw_row, rel=FOLD_REL, max_amb=6):
    """Every value row that quantising ``raw_row`` to MXFP4 may give when
    the value is computed in float32 (relative accuracy ``rel``): per block
    of 32, each E8M0 scale that a block maximum within rel of the exact one
    selects, and under each scale, both E2M1 neighbours of every element
    within rel of a rounding boundary.  Rounding is monotone, so the
    candidates are the roundings of the value moved by -rel and +rel.  At
    most 2**max_amb rows."""
    from oracle.formats import MX_BLOCK, _round_e2m1, e2m1_to_f64, mxfp4_quantize
    x = np.asarray(raw_row, np.float64)
    rows = [mxfp4_quantize(x)[2]]

    def code_of(amax):
        if amax <= 0:
            return 0
        _, e = np.frexp(amax)
        return int(np.clip(e - 1 - 2 + 127, 0, 254))

    for blk in range(x.size // MX_BLOCK):
        sl = slice(blk * MX_BLOCK, (blk + 1) * MX_BLOCK)
        xb = x[sl]
        amax = float(np.abs(xb).max())
        variants = []
        for code in sorted({code_of(amax * (1 - rel)), code_of(amax), code_of(amax * (1 + rel))}):
            scale = np.ldexp(1.0, code - 127)
            y = xb / scale
            lo = e2m1_to_f64(_round_e2m1(np.abs(y) * (1 - rel)))
            hi = e2m1_to_f64(_round_e2m1(np.abs(y) * (1 + rel)))
            vs = [lo.copy()]
            for i in np.where(lo != hi)[0]:
                vs += [v.copy() for v in vs]
                for v in vs[len(vs) // 2:]:
                    v[i] = hi[i]
            variants += [np.sign(y) * v * scale for v in vs]
        uniq = []
        for v in variants:
            if not any(np.array_equal(v, u) for u in uniq):
                uniq.append(v)
        if len(uniq) > 1:
            assert len(rows) * len(uniq) <= 2 ** max_amb, "too many ambiguous roundings in one key"
            new = []
            for r in rows:
                for v in uniq:
                    r2 = r.copy()
                    r2[sl] = v
                    new.append(r2)
            rows = new
    return rows


def ambiguous_mxfp4_keys(raw_rows, ids, rel=FOLD_REL):
    """{id: alternative value rows} for layer-produced MXFP4 keys whose
    stored codes or scales are not settled by float32 accuracy."""
    out = {}
    for s, raw in zip(ids, raw_rows):
        alts = mxfp4_alternatives(raw, rel)
        if len(alts) > 1:
            out[int(s)] = alts
    return out


def bf16_score_intervals(scores, err, bounds=None):
    """(lo, hi): the bfloat16 scores a float32 evaluation may round to, per
    entry.  ``scores`` are the exact (float64, unrounded) scores, ``err``
    their float32 evaluation error bounds, ``bounds`` ({id: (lo, hi)})
    widens entries whose key is only known within its rounding
    alternatives.  Rounding to bf16 is monotone, so the evaluated score
    within [s - e, s + e] rounds into [bf16(s - e), bf16(s + e)]."""
    from oracle.formats import round_to_bf16
    s = np.asarray(scores, np.float64)
    e = np.asarray(err, np.float64)
    lo, hi = s - e, s + e
    for i, (a, b) in (bounds or {}).items():
        if i < len(s):
            lo[i], hi[i] = a - e[i], b + e[i]
    return round_to_bf16(lo), round_to_bf16(hi)


def topk_check_intervals(gpu_ids, gpu_cnt, k, lo, hi):
    """Exact top-k check over scores known within intervals [lo, hi] (the
    bf16 scores): the GPU set S must be the top-k, ties to the lower id, of
    some scores within the intervals.  The most favourable choice is hi on S
    and lo elsewhere, so S is valid iff every pair i in S, j outside has
    hi_i > lo_j, or hi_i == lo_j and i < j.  Returns (ok, n_uncertain,
    message), n_uncertain counting the members of S whose interval is not a
    single value."""
    lo, hi = np.asarray(lo, np.float64), np.asarray(hi, np.float64)
    n = len(lo)
    gpu = np.asarray(gpu_ids)[:int(gpu_cnt)]
    if len(gpu) != min(k, n):
        return False, 0, f"count {len(gpu)} != {min(k, n)}"
    if len(gpu) and (np.any(np.diff(gpu) <= 0) or gpu.min() < 0 or gpu.max() >= n):
        return False, 0, "gpu ids not strictly ascending within the visible range"
    inside = np.zeros(n, bool)
    inside[gpu] = True
    if inside.all() or not inside.any():
        return True, 0, ""
    m = hi[inside].min()
    out_lo = lo[~inside]
    if out_lo.max() > m:
        j = int(np.where(~inside)[0][np.argmax(out_lo)])
        return False, 0, f"entry {j} (score >= {lo[j]}) outranks a selected entry (score <= {m})"
    at_m_in = np.where(inside & (hi == m))[0]
    at_m_out = np.where(~inside & (lo == m))[0]
    if at_m_out.size and at_m_in.max() > at_m_out.min():
        return False, 0, f"tie at {m}: selected id {at_m_in.max()} above unselected id {at_m_out.min()}"
    return True, int(np.count_nonzero(lo[inside] != hi[inside])), ""


def check_selection(ids, cnt, k, ref, err, bounds=None, score_dtype="f32"):
    """The selection rule for one query.  ``ref`` is the oracle's answer
    (sel, scores, scores_raw), ``err`` its score_error_bound (array or lazy
    function), ``bounds`` the score bounds of keys with several valid
    roundings.  float32 scores: topk_check_bounds; bf16 scores:
    topk_check_intervals over the bf16 roundings of the float32 error
    intervals.  Returns (ok, swapped, message), swapped true when the GPU
    set differs from the oracle's (its attention must then be compared
    with the oracle's on the GPU set)."""
    if score_dtype != "bf16":
        return topk_check_bounds(ids, cnt, ref["sel"], ref["scores"], k, bounds or {}, err=err)
    e = err() if callable(err) else err
    lo, hi = bf16_score_intervals(ref["scores_raw"], e, bounds)
    ok, _, msg = topk_check_intervals(ids, cnt, k, lo, hi)
    gpu = np.asarray(ids)[:int(cnt)]
    return ok, int(not np.array_equal(gpu, ref["sel"])), msg


def gpu_entries(state, b, sl, kvk):
    """Main-cache rows sl of sequence b of a device state, as float64 (the
    576-byte FP8 + BF16 rows decoded with their scales)."""
    from oracle.formats import Stored
    import torch
    if kvk == "fp8bf16":
        codes = state.kv_cache[b, sl].cpu().numpy()
        sc = state.kv_scale[b, sl].cpu().numpy()
        return Stored(codes, "fp8bf16", sc).all()
    return state.kv_cache[b, sl].detach().to(torch.float64).cpu().numpy()


def assert_entry_close(got, ref, kvk, what):
    """Produced main entries: with the FP8 + BF16 entry, the e4m3 part
    within one quantum of the oracle's value everywhere (the float32 value
    may sit on a rounding tie, and the scale may differ by float32 rounding)
    with at most 2 % of the codes flipped, and the bf16 part within the bf16
    tolerance; other formats: assert_close."""
    got = np.atleast_2d(np.asarray(got, np.float64))
    ref = np.atleast_2d(np.asarray(ref, np.float64))
    if kvk != "fp8bf16":
        return assert_close(got, ref, kvk, what)
    from oracle.formats import FP8_DIMS
    g8, r8 = got[:, :FP8_DIMS], ref[:, :FP8_DIMS]
    scale = np.abs(r8).max(axis=1, keepdims=True) / 448.0
    step = np.abs(r8) / 8 + scale * 2.0 ** -9
    assert np.all(np.abs(g8 - r8) <= step * 1.0001 + 1e-30), f"{what}: e4m3 part beyond one quantum"
    flips = np.abs(g8 - r8) > 1e-5 * np.maximum(np.abs(r8).max(axis=1, keepdims=True), 1e-30)
    assert flips.mean() <= 0.02, f"{what}: {flips.mean():.3f} e4m3 codes differ"
    return assert_close(got[:, FP8_DIMS:], ref[:, FP8_DIMS:], "bf16", what + " (bf16 part)")


def rel_err_rows(gpu, ref):
    """Per-row relative errors (rows = last axis vectors)."""
    g = np.asarray(gpu, np.float64).reshape(-1, np.shape(gpu)[-1])
    r = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    rowmax = np.abs(r).max(axis=1)
    floor = 1e-3 * np.median(rowmax) if rowmax.size else 0.0
    den = np.maximum(rowmax, max(floor, 1e-30))
    return np.abs(g - r).max(axis=1) / den


def assert_close(gpu, ref, kind, what=""):
    tol = TOL[kind]
    e = rel_err_rows(gpu, ref)
    worst = int(np.argmax(e)) if e.size else 0
    maxabs = float(np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64)).max())
    assert e.size == 0 or e.max() <= tol, (
        f"{what}: worst row {worst} rel err {e.max():.3e} > {tol} (max-abs {maxabs:.3e})")
    return float(e.max()) if e.size else 0.0, maxabs


def bf16_bits_to_f32(bits):
    return (np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
