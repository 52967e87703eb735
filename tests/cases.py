"""Test-side helpers that re-slice generated inputs (no method arithmetic).

``decode_from_prefill`` turns a prefill workload into the decode-step inputs
of one later token, so that prefill(n) + decode steps can be checked against
prefill(n + d) on identical token data (the continuation check the book
recommends in ch. 13).
"""

import numpy as np

from oracle.formats import f64_to_bf16_bits


def _bits(x, kind):
    if kind == "bf16":
        return f64_to_bf16_bits(x)
    return np.asarray(x, dtype=np.float32)


def prefix_case(pre, T):
    """The same prefill workload cut to its first T chunk tokens."""
    g = dict(pre)
    g["T"] = T
    for n in ("ca", "za", "cb", "zb", "ica", "iza", "icb", "izb", "q", "q_idx", "w_idx"):
        if n in g and g[n] is not None:
            g[n] = g[n][:, :T]
    g["win"] = pre["win"][:, :pre["n_win"] - 1 + T]
    return g


def decode_from_prefill(pre, T_done, kv_new, idx_new, t, extra_kv=(), extra_idx=()):
    """Decode inputs for the token at position t, after a prefill of the first
    T_done chunk tokens produced entries ``kv_new`` / ``idx_new`` (float64,
    rounded to storage) and later decode steps produced ``extra_*`` entries.
    Only batch row 0 is used."""
    m, c, n_win = pre["m"], pre["c"], pre["n_win"]
    pos0 = int(pre["pos0"])
    kvk = pre["kv_dtype"]
    n_old = int(pre["n_entries"][0])
    kv_rows = list(kv_new) + list(extra_kv)
    n_have = n_old + len(kv_rows)
    E_cap = max(pre["E_cap"], n_have + 1)
    g = {k: pre[k] for k in ("kind", "H", "c", "m", "n_win", "overlap", "vis", "scale",
                             "kv_dtype", "k", "idx_dtype", "sink", "bias_a", "bias_b")}
    g.update(B=1, E_cap=E_cap)
    g["pos"] = np.array([t], dtype=np.int64)
    g["n_entries"] = np.array([n_have], dtype=np.int32)
    kv = np.zeros((1, E_cap, c), dtype=pre["kv_cache"].dtype)
    kv[0, :n_old] = pre["kv_cache"][0, :n_old]
    if kv_rows:
        kv[0, n_old:n_have] = _bits(np.array(kv_rows), kvk)
    g["kv_cache"] = kv
    tail_len = 2 * m if pre["overlap"] else m
    g["tail_pos0"] = np.array([t - tail_len], dtype=np.int64)
    lo, hi = t - tail_len - pos0, t - pos0
    assert lo >= 0, "tail reaches before the chunk"
    streams = ("ca", "za", "cb", "zb") if pre["overlap"] else ("ca", "za")
    for s in streams:
        g["tail_" + s] = pre[s][:, lo:hi]
        g["new_" + s] = pre[s][:, hi]
    w0 = t - (n_win - 1) - (pos0 - (n_win - 1))
    g["win_hist"] = pre["win"][:, w0:w0 + n_win - 1]
    g["x_new"] = pre["win"][:, w0 + n_win - 1]
    g["q"] = pre["q"][:, hi]
    if pre["kind"] == "csa":
        d_I = pre["d_I"]
        g.update(H_I=pre["H_I"], d_I=d_I, ibias_a=pre["ibias_a"], ibias_b=pre["ibias_b"])
        ik = np.zeros((1, E_cap, d_I), dtype=pre["idx_cache"].dtype)
        ik[0, :n_old] = pre["idx_cache"][0, :n_old]
        idx_rows = list(idx_new) + list(extra_idx)
        if idx_rows:
            ik[0, n_old:n_have] = _bits(np.array(idx_rows), pre["idx_dtype"])
        g["idx_cache"] = ik
        g["idx_scale"] = None
        for s in ("ca", "za", "cb", "zb"):
            g["tail_i" + s] = pre["i" + s][:, lo:hi]
            g["new_i" + s] = pre["i" + s][:, hi]
        g["q_idx"] = pre["q_idx"][:, hi]
        g["q_scale"] = None
        g["w_idx"] = pre["w_idx"][:, hi]
    return g
