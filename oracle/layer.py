"""Layer-level oracle: a decode step and a prefill chunk (test infrastructure).

A layer step is the four parts of the hot path in the pages' order: fold any
block that has completed into a compressed entry, score the visible entries
with the lightning indexer, keep the top-k (CSA only), and attend over the
selected (CSA) or all visible (HCA) entries together with the sliding window
and the sink ("2026 DeepSeek-V4" note, ``csa()`` and ``hca()`` in "Key design
1" / "Key design 2"; "DeepSeek-V4" book ch. 5-7).

The cache is split as the pages describe it ("DeepSeek-V4" book ch. 5 "What
is retained during decode"): a classical cache of completed entries plus
bounded state (window rows and the compression tail).  Here the state is
given by position (``tail_*`` arrays hold tokens ``tail_pos0 ..``); how the
HIP path lays it out in memory is its own business.

With ``norm_rope`` set in a case, the steps on either side of the core
attention are included ("DeepSeek-V4" book ch. 7 "Query and KV
normalization", "Partial rotary position embeddings", "Why the output is
de-rotated"; see position.py): produced entries and window rows are
normalised and rotated at their positions before storage, the query at its
position, and the output is rotated back by the query's rotation.
"""

import numpy as np

from . import csa
from . import position as P
from .formats import Stored


class CacheView:
    """Rows 0..n_base-1 from a stored cache, rows n_base.. from ``extra``
    (float64 rows the step itself produced, already rounded to storage)."""

    def __init__(self, base: Stored, n_base, extra=None):
        self.base = base
        self.n_base = int(n_base)
        self.extra = np.zeros((0, base.width)) if extra is None else np.asarray(extra)

    def __len__(self):
        return self.n_base + len(self.extra)

    def rows(self, idx):
        if isinstance(idx, slice):
            idx = np.arange(*idx.indices(len(self)))
        idx = np.asarray(idx, dtype=np.int64)
        out = np.empty((idx.shape[0], self.base.width))
        lo = idx < self.n_base
        if lo.any():
            out[lo] = self.base.rows(idx[lo])
        if (~lo).any():
            out[~lo] = self.extra[idx[~lo] - self.n_base]
        return out


def _store_key(x, kind):
    if kind == "e4m3":
        return csa.e4m3_quantize_rows(x[None, :])[0][0]
    return csa.store_as(x, kind)


def _act(g):
    """Storage kind of the activations (token streams, window rows,
    queries): that of the cache, except under the mixed FP8 + BF16 cache,
    whose activations stay bf16."""
    k = g["kv_dtype"]
    return "bf16" if k == "fp8bf16" else k


def _dec(x, kind, scale=None):
    return Stored(x, kind, scale).all()


def _nr(g):
    """(q scale, KV scale, eps, inverse frequencies) when the layer
    normalises and rotates its queries and KV vectors, else None."""
    if not g.get("norm_rope"):
        return None
    return (g["q_norm_w"], g["kv_norm_w"], float(g["norm_eps"]), g["rope_inv_freq"])


def _prep_kv(nr, x, pos):
    """A produced KV vector (entry or window row) as stored for attention."""
    return x if nr is None else P.prepare(x, nr[1], nr[2], pos, nr[3])


def _prep_q(nr, q, t, act):
    """The query the core attention reads: prepared, then held in the
    activation format like every input of the core attention."""
    return q if nr is None else csa.store_as(P.prepare(q, nr[0], nr[2], t, nr[3]), act)


def _post(nr, o, t):
    return o if nr is None else P.derotate(o, t, nr[3])


# ---------------------------------------------------------------------------
# decode step: one new token per sequence
# ---------------------------------------------------------------------------

def decode_step(case, b, selected=None):
    """One decode step of sequence b of a decode workload ``case``.

    The new token at t = pos[b] is appended to the state, every block that a
    query at t may read but that is not yet in the cache is folded, and the
    query is answered.  Returns a dict with o [H][c], lse [H], and for CSA the
    selected ids and the visible scores (as selected on, and before any
    rounding: scores_raw), plus the folded entries.
    """
    g = case
    t = int(g["pos"][b])
    m, c = g["m"], g["c"]
    kvk, idk = g["kv_dtype"], g["idx_dtype"]
    act = _act(g)
    nr = _nr(g)
    n_have = int(g["n_entries"][b])
    need = t // m if g["vis"] == csa.VIS_PRIOR_BLOCKS else (t + 1) // m
    p0 = int(g["tail_pos0"][b])

    def stream(name, d_kind):
        """Tokens tail_pos0 .. t of one compressor stream as float64."""
        hist = _dec(g["tail_" + name][b], d_kind)
        new = _dec(g["new_" + name][b][None], d_kind)
        return np.concatenate([hist, new], axis=0)

    folded_kv, folded_idx, folded_idx_raw = [], [], []
    if need > n_have:
        overlap = g["overlap"]
        s = {n: stream(n, act) for n in (("ca", "za", "cb", "zb") if overlap else ("ca", "za"))}
        si = {}
        if g["kind"] == "csa":
            si = {n: stream("i" + n, act) for n in ("ca", "za", "cb", "zb")}
        for e in range(n_have, need):
            a = slice(m * e - p0, m * e + m - p0)
            if a.start < 0 or a.stop > t - p0 + 1:
                raise ValueError("tail does not hold the block to fold")
            use_prev = overlap and e > 0
            if use_prev:
                pb = slice(m * (e - 1) - p0, m * e - p0)
                if pb.start < 0:
                    raise ValueError("tail does not hold the previous block")
                ent = csa.compress_entry(s["ca"][a], s["za"][a], g["bias_a"],
                                         s["cb"][pb], s["zb"][pb], g["bias_b"])
            else:
                ent = csa.compress_entry(s["ca"][a], s["za"][a], g["bias_a"])
            folded_kv.append(csa.store_as(_prep_kv(nr, ent, P.entry_position(e, m)), kvk))
            if g["kind"] == "csa":
                if use_prev:
                    ik = csa.compress_entry(si["ca"][a], si["za"][a], g["ibias_a"],
                                            si["cb"][pb], si["zb"][pb], g["ibias_b"])
                else:
                    ik = csa.compress_entry(si["ca"][a], si["za"][a], g["ibias_a"])
                folded_idx.append(_store_key(ik, idk))
                folded_idx_raw.append(ik)
    n_total = max(n_have, need)
    kv = CacheView(Stored(g["kv_cache"][b], kvk, None if g.get("kv_scale") is None else g["kv_scale"][b]),
                   n_have, np.array(folded_kv) if folded_kv else None)

    # the window ring holds rows as stored: with normalisation and rotary
    # positions on, the history rows are already prepared and the new
    # token's row is prepared (and rounded to storage) by the step
    win_hist = _dec(g["win_hist"][b], act)  # positions t-(n_win-1) .. t-1
    x_new = _dec(g["x_new"][b][None], act)
    if nr is not None:
        x_new = csa.store_as(_prep_kv(nr, x_new, t), act)
    win_all = np.concatenate([win_hist, x_new], axis=0)
    wp0 = t - win_hist.shape[0]

    def win_rows(pos):
        return win_all[np.asarray(pos) - wp0]

    q = _prep_q(nr, _dec(g["q"][b], act), t, act)
    sink = None if g["sink"] is None else np.asarray(g["sink"], np.float64)
    # (folded_idx_raw: the indexer keys before rounding to storage, for tests
    # that must know which stored codes a rounding decision settles)
    out = {"folded_kv": folded_kv, "folded_idx": folded_idx, "folded_idx_raw": folded_idx_raw}
    if g["kind"] == "csa":
        keys = CacheView(Stored(g["idx_cache"][b], idk,
                                None if g["idx_scale"] is None else g["idx_scale"][b]),
                         n_have, np.array(folded_idx) if folded_idx else None)
        qi = _dec(g["q_idx"][b], idk, None if g["q_scale"] is None else g["q_scale"][b])
        w = np.asarray(g["w_idx"][b], np.float64)
        o, lse, sel, scores, raw = csa.csa_query(q, qi, w, t, kv, keys, n_total, win_rows, sink,
                                                 m, g["k"], g["n_win"], g["scale"], g["vis"],
                                                 selected=selected, score_dtype=g.get("score_dtype", "f32"),
                                                 return_raw=True)
        out.update(o=_post(nr, o, t), lse=lse, sel=sel, scores=scores, scores_raw=raw)
    else:
        o, lse = csa.hca_query(q, t, kv, n_total, win_rows, sink, m, g["n_win"], g["scale"],
                               g["vis"])
        out.update(o=_post(nr, o, t), lse=lse)
    return out


# ---------------------------------------------------------------------------
# prefill chunk
# ---------------------------------------------------------------------------

def prefill_entries(case, b, raw=False):
    """Compress a prefill chunk of sequence b into new cache entries (main KV
    and, for CSA, indexer keys), rounded to their storage formats.  With
    raw=True the indexer keys before rounding are returned as a third value."""
    g = case
    m = g["m"]
    kvk, idk = g["kv_dtype"], g["idx_dtype"]
    act = _act(g)
    nr = _nr(g)
    d = lambda n: _dec(g[n][b], act)  # noqa: E731
    if g["overlap"]:
        first = int(g["pos0"]) == 0
        ent = csa.compress(d("ca"), d("za"), m, g["bias_a"], d("cb"), d("zb"), g["bias_b"],
                           None if first else d("prev_cb"), None if first else d("prev_zb"))
    else:
        ent = csa.compress(d("ca"), d("za"), m, g["bias_a"])
    first = int(g["pos0"]) // m  # the chunk's first entry
    if nr is not None:
        ent = _prep_kv(nr, ent, P.entry_position(first + np.arange(len(ent)), m))
    kv_new = csa.store_as(ent, kvk)
    idx_new = None
    if g["kind"] == "csa":
        first = int(g["pos0"]) == 0
        ik = csa.compress(d("ica"), d("iza"), m, g["ibias_a"], d("icb"), d("izb"), g["ibias_b"],
                          None if first else d("prev_icb"), None if first else d("prev_izb"))
        if idk == "e4m3":
            idx_new = csa.e4m3_quantize_rows(ik)[0]
        else:
            idx_new = csa.store_as(ik, idk)
    if raw:
        return kv_new, idx_new, (ik if g["kind"] == "csa" else None)
    return kv_new, idx_new


def prefill_query(case, b, i, kv_new, idx_new, selected=None):
    """Answer chunk query i (position pos0 + i) of sequence b, given the
    chunk's compressed entries from ``prefill_entries``."""
    g = case
    m = g["m"]
    kvk, idk = g["kv_dtype"], g["idx_dtype"]
    t = int(g["pos0"]) + i
    n_have = int(g["n_entries"][b])
    kv = CacheView(Stored(g["kv_cache"][b], kvk, None if g.get("kv_scale") is None else g["kv_scale"][b]),
                   n_have, kv_new)
    n_total = n_have + len(kv_new)
    wp0 = int(g["pos0"]) - (g["n_win"] - 1)
    act = _act(g)
    nr = _nr(g)
    wstore = Stored(g["win"][b], act)

    def win_rows(pos):
        pos = np.asarray(pos)
        rows = wstore.rows(pos - wp0)
        # with normalisation and rotary positions on, the chunk's window rows
        # are prepared at their positions and stored for the attention
        return rows if nr is None else csa.store_as(_prep_kv(nr, rows, pos), act)

    q = _prep_q(nr, _dec(g["q"][b][i], act), t, act)
    sink = None if g["sink"] is None else np.asarray(g["sink"], np.float64)
    if g["kind"] == "csa":
        keys = CacheView(Stored(g["idx_cache"][b], idk,
                                None if g.get("idx_scale") is None else g["idx_scale"][b]),
                         n_have, idx_new)
        qi = _dec(g["q_idx"][b][i], idk,
                  None if g.get("q_scale") is None else g["q_scale"][b][i])
        w = np.asarray(g["w_idx"][b][i], np.float64)
        o, lse, sel, scores, raw = csa.csa_query(q, qi, w, t, kv, keys, n_total, win_rows, sink,
                                                 m, g["k"], g["n_win"], g["scale"], g["vis"],
                                                 selected=selected, score_dtype=g.get("score_dtype", "f32"),
                                                 return_raw=True)
        return {"o": _post(nr, o, t), "lse": lse, "sel": sel, "scores": scores, "scores_raw": raw}
    o, lse = csa.hca_query(q, t, kv, n_total, win_rows, sink, m, g["n_win"], g["scale"],
                           g["vis"])
    return {"o": _post(nr, o, t), "lse": lse}


# ---------------------------------------------------------------------------
# tiny whole-context case (scalar compression logits)
# ---------------------------------------------------------------------------

def tiny_entries(case):
    """Compress the whole context of the tiny case: one scalar logit w . x per
    token, a softmax over each m-token block, entry = weighted sum of the
    block (no overlap, no bias); the indexer keys the same way from their own
    raw keys."""
    g = case
    x = g["x"][0].astype(np.float64)
    xi = g["x_idx"][0].astype(np.float64)
    kv = csa.compress(x, csa.scalar_logits(x, g["w_cmp"]), g["m"])
    keys = csa.compress(xi, csa.scalar_logits(xi, g["w_cmp_idx"]), g["m"])
    return csa.store_as(kv, "f32"), csa.store_as(keys, "f32")


def tiny_query(case, i, kv, keys, selected=None):
    g = case
    t = int(g["q_pos"][0][i])
    x = g["x"][0].astype(np.float64)
    kvv = CacheView(Stored(np.zeros((0, kv.shape[1]), np.float32), "f32"), 0, kv)
    kk = CacheView(Stored(np.zeros((0, keys.shape[1]), np.float32), "f32"), 0, keys)
    return csa.csa_query(g["q"][0][i].astype(np.float64), g["q_idx"][0][i].astype(np.float64),
                         g["w_idx"][0][i].astype(np.float64), t, kvv, kk, len(kv),
                         lambda pos: x[np.asarray(pos)], np.asarray(g["sink"], np.float64),
                         g["m"], g["k"], g["n_win"], g["scale"], g["vis"], selected=selected)
