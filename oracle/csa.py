"""Oracle for the CSA / HCA hybrid-attention layer (test infrastructure only).

Plain float64 NumPy, one formula per function, written from the pages:

* "DeepSeek-V4" book, ch. 5 "How CSA Compresses Memory", ch. 6 "How CSA
  Selects and Reads Memory", ch. 7 "HCA, Local Attention, and Position",
  ch. 8 "A Cost Model for Long Context", ch. 13 (inference framework).
* "2026 DeepSeek-V4" research note, "Method Deep Dive" (visible-set sizes and
  the configuration table), "Key design 1" (CSA compressor, indexer and top-k
  equations) and "Key design 2" (HCA compressor equation).

Readings where the pages are silent or garbled (each listed in the design
notes): visibility is s < floor(t/m) for a query at 0-based position t; the
window holds positions max(0, t-n_win+1) .. t including the query's own token;
compressed rows and window rows share one softmax together with the sink;
the attention scale is passed in (1/sqrt(c) in every workload); the top-k
keeps the k largest scores, the lower entry id winning a tie, and returns
ids in ascending order.

Nothing here is blocked, fused or reordered beyond what the formulas state.
Large arrays are only ever decoded row-subset by row-subset (``Stored.rows``).
"""

import math

import numpy as np

from .formats import FP8_DIMS, Stored, mxfp4_quantize, round_to_bf16

VIS_PRIOR_BLOCKS = 0  # entry s visible to a query at t iff s < floor(t / m)
VIS_COMPLETED = 1  # entry s visible iff s < floor((t + 1) / m)


# ---------------------------------------------------------------------------
# entry counts and visibility
# ---------------------------------------------------------------------------

def entry_count(n, m):
    """Completed entries and pending tail after n tokens at compression m.

    A trailing fragment shorter than m produces no completed entry; it stays
    in the state cache.  ("DeepSeek-V4" book ch. 7 "HCA's compressor": 10**6
    tokens give 7,812 complete blocks and 64 remaining tokens; ch. 13: a
    1,000-token prefix gives 250 CSA entries and 7 HCA entries plus a
    104-token tail.)
    """
    return n // m, n % m


def visible_entries(t, m, n_entries, vis=VIS_PRIOR_BLOCKS):
    """Number of compressed entries a query at position t may read.

    A query uses only preceding completed blocks ("DeepSeek-V4" book ch. 5
    "When an entry becomes available"); the same mask applies to the indexer's
    top-k.  The printed condition is garbled; the default reading is
    s < floor(t/m).  ``VIS_COMPLETED`` also admits the block the query itself
    completes.
    """
    lim = t // m if vis == VIS_PRIOR_BLOCKS else (t + 1) // m
    return max(0, min(int(n_entries), lim))


def window_positions(t, n_win):
    """Positions of the uncompressed sliding window of a query at t.

    Up to n_win recent uncompressed entries ("DeepSeek-V4" book ch. 7 "The
    sliding window"), read as positions max(0, t-n_win+1) .. t.
    """
    return np.arange(max(0, t - n_win + 1), t + 1)


# ---------------------------------------------------------------------------
# a1: compressor
# ---------------------------------------------------------------------------

def _broadcast_logits(z, c):
    z = np.asarray(z, dtype=np.float64)
    if z.shape[-1] == 1:
        z = np.broadcast_to(z, z.shape[:-1] + (c,))
    return z


def compress_entry(ca, za, ba, cb=None, zb=None, bb=None):
    """One compressed entry from its source tokens, per coordinate.

    ca, za: [m][c] content and logits of the current block (branch a);
    cb, zb: [m][c] of the previous block through branch b, or None.
    ba, bb: [m][c] positional biases (None = 0).

    For each coordinate r the logits Z[j, r] + B[j, r] of all source
    positions j (current block via a, previous block via b) go through one
    softmax across the source positions, independently per coordinate, and the
    entry is the weighted sum of the contents ("2026 DeepSeek-V4" note, "Key
    design 1" equation; "DeepSeek-V4" book ch. 5 "One weight distribution per
    coordinate").  A missing previous block contributes zero content with
    logit -inf, i.e. no weight (book ch. 5, start-of-sequence rule).  Without
    branch b this is the HCA compressor ("Key design 2" equation).
    """
    ca = np.asarray(ca, dtype=np.float64)
    m, c = ca.shape
    la = _broadcast_logits(za, c) + (0.0 if ba is None else np.asarray(ba, np.float64))
    logits = [la]
    contents = [ca]
    if cb is not None:
        lb = _broadcast_logits(zb, c) + (0.0 if bb is None else np.asarray(bb, np.float64))
        logits.append(lb)
        contents.append(np.asarray(cb, dtype=np.float64))
    L = np.concatenate(logits, axis=0)  # [sources][c]
    C = np.concatenate(contents, axis=0)
    mx = L.max(axis=0, keepdims=True)
    e = np.exp(L - mx)
    S = e / e.sum(axis=0, keepdims=True)  # softmax across source positions
    return (S * C).sum(axis=0)


def compress(content_a, logits_a, m, bias_a=None,
             content_b=None, logits_b=None, bias_b=None,
             prev_content_b=None, prev_logits_b=None):
    """Entries for a token chunk that starts on a block boundary.

    content_*: [T][c]; logits_*: [T][c] or [T][1] (one scalar per token,
    shared by all coordinates); T % m == 0.  Entry i of the chunk draws on
    chunk tokens m*i .. m*i+m-1 through branch a and, when branch b is given,
    on tokens m*(i-1) .. m*i-1 through branch b ("DeepSeek-V4" book ch. 5
    "Which positions enter a compressed block").  For i = 0 the previous block
    comes from ``prev_*_b`` ([m][c]); if those are None the chunk starts the
    sequence and entry 0 has no previous block.
    """
    content_a = np.asarray(content_a, dtype=np.float64)
    T, c = content_a.shape
    if T % m:
        raise ValueError("chunk length must be a multiple of m")
    overlap = content_b is not None
    out = np.empty((T // m, c))
    for i in range(T // m):
        blk = slice(m * i, m * i + m)
        cb = zb = None
        if overlap:
            if i > 0:
                prev = slice(m * (i - 1), m * i)
                cb, zb = content_b[prev], logits_b[prev]
            elif prev_content_b is not None:
                cb, zb = prev_content_b, prev_logits_b
        out[i] = compress_entry(content_a[blk], logits_a[blk], bias_a,
                                cb, zb, bias_b if cb is not None else None)
    return out


def scalar_logits(x, w):
    """Per-token scalar compression logit w . x_t (the one-logit-per-token
    form used by the tiny fp32 workload; broadcast over coordinates)."""
    return (np.asarray(x, np.float64) @ np.asarray(w, np.float64))[:, None]


# ---------------------------------------------------------------------------
# a2: lightning indexer
# ---------------------------------------------------------------------------

def index_scores(q_idx, w_idx, keys):
    """I[s] = sum_h w[h] * ReLU(q[h] . K[s]) for every row s of ``keys``.

    q_idx [H_I][d_I], w_idx [H_I] (signed: the head weights are an
    unconstrained linear projection), keys [S][d_I].  ("2026 DeepSeek-V4"
    note, "Key design 1" indexer equation; "DeepSeek-V4" book ch. 6 "The index
    score".)
    """
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)
    dots = K @ q.T  # [S][H_I]: q_h . K_s
    return np.maximum(dots, 0.0) @ w


def index_scores_stored(q_idx, w_idx, keys: Stored, n, chunk=65536):
    """index_scores over rows 0..n-1 of a stored key cache, decoding it
    ``chunk`` rows at a time (each score is independent of the others)."""
    out = np.empty(n)
    for s0 in range(0, n, chunk):
        s1 = min(n, s0 + chunk)
        out[s0:s1] = index_scores(q_idx, w_idx, keys.rows(slice(s0, s1)))
    return out


# ---------------------------------------------------------------------------
# a3: top-k
# ---------------------------------------------------------------------------

def topk_select(scores, k):
    """Ids of the k largest scores (all of them if fewer than k), ascending.

    C_t = TopK_k(I_t,:) ("Key design 1" equation).  When fewer than k entries
    are eligible all are kept ("DeepSeek-V4" book ch. 6 "Top-k is a budget over
    compressed entries").  Ties, which the pages leave open, go to the lower
    entry id.
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    ids = np.arange(n)
    order = np.lexsort((ids, -scores))  # by score descending, then id ascending
    return np.sort(order[:min(k, n)])


# ---------------------------------------------------------------------------
# a4 / a5 / a6: shared-KV attention with window and sink
# ---------------------------------------------------------------------------

def attend(q, rows, sink=None, scale=None):
    """Shared key-value MQA over ``rows`` with an attention sink.

    q [H][c] query heads; rows [R][c]: every row serves as both key and value
    for all heads ("DeepSeek-V4" book ch. 6 "Shared key-value MQA").
    Compressed rows and window rows arrive here already concatenated and share
    one softmax ("2026 DeepSeek-V4" note, ``concat(selected, local_kv)``; book
    ch. 7 "The sliding window").  The sink logit z'_h adds exp(z'_h) to the
    denominator and nothing to the numerator (book ch. 7 "Attention sinks").

    Returns o [H][c] and lse [H] = log(sum_j exp(l_hj) + exp(z'_h)).
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    H, c = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(c)
    logits = scale * (q @ rows.T)  # [H][R]
    z = np.full(H, -np.inf) if sink is None else np.asarray(sink, np.float64)
    M = np.maximum(logits.max(axis=1) if rows.shape[0] else np.full(H, -np.inf), z)
    e = np.exp(logits - M[:, None])
    denom = e.sum(axis=1) + np.exp(z - M)
    o = (e @ rows) / denom[:, None]
    lse = M + np.log(denom)
    return o, lse


def merge_partials(parts, sink=None):
    """Combine attention partials computed over disjoint row sets.

    Each part is (mx [H], l [H], acc [H][c]) with l = sum exp(logit - mx) and
    acc = sum exp(logit - mx) * row.  The result equals one softmax over the
    union of the rows plus the sink (used to pin split/merge invariance).
    """
    mx = np.max(np.stack([p[0] for p in parts]), axis=0)
    if sink is not None:
        mx = np.maximum(mx, sink)
    l = sum(p[1] * np.exp(p[0] - mx) for p in parts)
    acc = sum(p[2] * np.exp(p[0] - mx)[:, None] for p in parts)
    if sink is not None:
        l = l + np.exp(np.asarray(sink) - mx)
    return acc / l[:, None], mx + np.log(l)


def attend_partial(q, rows, scale):
    """(mx, l, acc) of one row subset, for ``merge_partials``."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    logits = scale * (q @ rows.T)
    mx = logits.max(axis=1)
    e = np.exp(logits - mx[:, None])
    return mx, e.sum(axis=1), e @ rows


# ---------------------------------------------------------------------------
# one query of a layer
# ---------------------------------------------------------------------------

def csa_query(q, q_idx, w_idx, t, kv: Stored, keys: Stored, n_entries, win_rows,
              sink, m, k, n_win, scale, vis=VIS_PRIOR_BLOCKS, selected=None, score_dtype="f32",
              return_raw=False):
    """CSA for one query at position t.

    Score the visible compressed entries with the indexer, keep the top-k,
    and attend over the selected entries plus the window rows and the sink
    ("2026 DeepSeek-V4" note, "Key design 1"; "DeepSeek-V4" book ch. 6).
    ``win_rows(positions)`` returns the raw window rows.  ``selected`` may
    override the top-k set (used to evaluate attention on an equally valid
    set when two scores tie within rounding).  ``score_dtype="bf16"`` rounds
    the index scores to bfloat16 before the selection ("DeepSeek-V4" book
    ch. 16 "BF16 index scores"); ties, now frequent, still go to the lower
    entry id, and the rounded scores are returned.

    Returns (o [H][c], lse [H], selected ids, scores of the visible entries),
    and with return_raw the scores before any rounding as a fifth value.
    """
    n_vis = visible_entries(t, m, n_entries, vis)
    raw = index_scores_stored(q_idx, w_idx, keys, n_vis)
    scores = round_to_bf16(raw) if score_dtype == "bf16" else raw
    sel = topk_select(scores, k) if selected is None else np.asarray(selected)
    rows = np.concatenate([kv.rows(sel), win_rows(window_positions(t, n_win))], axis=0)
    o, lse = attend(q, rows, sink, scale)
    if return_raw:
        return o, lse, sel, scores, raw
    return o, lse, sel, scores


def hca_query(q, t, kv: Stored, n_entries, win_rows, sink, m, n_win, scale,
              vis=VIS_PRIOR_BLOCKS):
    """HCA for one query at t: dense attention over every visible compressed
    entry plus the window rows and the sink ("2026 DeepSeek-V4" note, "Key
    design 2"; "DeepSeek-V4" book ch. 7 "Dense attention over compressed
    history")."""
    n_vis = visible_entries(t, m, n_entries, vis)
    rows = np.concatenate([kv.rows(slice(0, n_vis)), win_rows(window_positions(t, n_win))],
                          axis=0)
    return attend(q, rows, sink, scale)


# ---------------------------------------------------------------------------
# storage rounding of produced entries
# ---------------------------------------------------------------------------

def store_as(x, kind):
    """Value of x after storage in ``kind``: "f32" or "bf16" (rounded to
    nearest-even once), "mxfp4" (OCP MX FP4, blocks of 32 along the last
    axis) or "fp8bf16" (the 576-byte entry: the first 448 coordinates e4m3
    with one scale per vector, the last 64 bf16)."""
    x = np.asarray(x, dtype=np.float64)
    if kind == "bf16":
        return round_to_bf16(x)
    if kind == "f32":
        return x.astype(np.float32).astype(np.float64)
    if kind == "mxfp4":
        return mxfp4_quantize(x)[2]
    if kind == "fp8bf16":
        head = e4m3_quantize_rows(x[..., :FP8_DIMS])[0]
        return np.concatenate([head, round_to_bf16(x[..., FP8_DIMS:])], axis=-1)
    raise ValueError(kind)


def e4m3_quantize_rows(x):
    """Quantise rows to OCP e4m3fn with one scale per row: scale = max|x|/448
    and code = nearest e4m3 value of x/scale, ties to even.  Returns the
    float64 values code*scale and the scales.  Used for indexer keys that the
    layer itself produces when the indexer cache is stored in fp8.  The scale
    is formed in float32, as it is stored.
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    scale = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = x / scale.astype(np.float64)[..., None]
    a = np.minimum(np.abs(y), 448.0)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    spacing = np.ldexp(1.0, np.maximum(e - 4, -9))  # 4 significant bits; subnormal step 2**-9
    r = np.rint(a / spacing) * spacing
    r = np.minimum(r, 448.0)
    return np.copysign(r, y) * scale.astype(np.float64)[..., None], scale
