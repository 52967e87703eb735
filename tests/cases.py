"""Test-side helpers that re-slice generated inputs (no method arithmetic of
their own: where a layer stores prepared window rows, they are prepared by
the oracle).

``decode_from_prefill`` turns a prefill workload into the decode-step inputs
of one later token, so that prefill(n) + decode steps can be checked against
prefill(n + d) on identical token data (the continuation check the book
recommends in ch. 13).
"""

import numpy as np
import torch

from oracle.formats import f64_to_bf16_bits


def _bits(x, kind):
    if kind == "bf16":
        return f64_to_bf16_bits(x)
    return np.asarray(x, dtype=np.float32)


def e4m3_codes_of(rows):
    """(codes, scales) of float64 rows that are e4m3 values times one float32
    scale per row with max |row| = 448 * scale (as the oracle's e4m3
    quantiser leaves them); an all-zero row has scale 1.  Pure re-encoding:
    every value divided by its scale is an e4m3 value, so torch's cast is
    exact here."""
    rows = np.asarray(rows, np.float64)
    amax = np.abs(rows).max(axis=-1)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    y = rows / scale.astype(np.float64)[..., None]
    codes = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn)
    back = codes.to(torch.float32).numpy().astype(np.float64)
    assert np.array_equal(back, y), "row is not an e4m3 row times its scale"
    return codes.view(torch.uint8).numpy(), scale


def fp8bf16_codes_of(rows):
    """(576-byte rows, float32 scales) of float64 rows that already are
    FP8 + BF16 entries (the first 448 values e4m3 times one scale, the last
    64 bf16 values): a pure re-encoding."""
    from oracle.formats import FP8_DIMS
    rows = np.asarray(rows, np.float64)
    codes, scale = e4m3_codes_of(rows[..., :FP8_DIMS])
    tail = f64_to_bf16_bits(rows[..., FP8_DIMS:]).astype(np.uint16)
    out = np.empty(rows.shape[:-1] + (576,), np.uint8)
    out[..., :FP8_DIMS] = codes
    out[..., FP8_DIMS:] = tail.view(np.uint8).reshape(rows.shape[:-1] + (128,))
    return out, scale


def mxfp4_codes_of(rows):
    """(packed codes, E8M0 scales) of float64 rows that already are MXFP4
    values (E2M1 values times a power-of-two scale per block of 32, as the
    oracle's quantiser leaves them): re-encoding them is exact."""
    import workloads
    rows = np.asarray(rows, np.float64)
    packed, scales = workloads.gen.mxfp4_rows(rows.astype(np.float32))
    from oracle.formats import mxfp4_decode
    assert np.array_equal(mxfp4_decode(packed, scales), rows), "row is not an MXFP4 row"
    return packed, scales


def prefix_case(pre, T):
    """The same prefill workload cut to its first T chunk tokens."""
    g = dict(pre)
    g["T"] = T
    for n in ("ca", "za", "cb", "zb", "ica", "iza", "icb", "izb", "q", "q_idx", "w_idx", "q_scale"):
        if n in g and g[n] is not None:
            g[n] = g[n][:, :T]
    g["win"] = pre["win"][:, :pre["n_win"] - 1 + T]
    return g


def decode_from_prefill(pre, T_done, kv_new, idx_new, t, extra_kv=(), extra_idx=(), b=0):
    """Decode inputs for sequence b's token at position t, after a prefill of
    the first T_done chunk tokens produced entries ``kv_new`` / ``idx_new``
    (float64, rounded to storage) and later decode steps produced ``extra_*``
    entries.  The result is a one-sequence decode workload."""
    m, c, n_win = pre["m"], pre["c"], pre["n_win"]
    pos0 = int(pre["pos0"])
    kvk = pre["kv_dtype"]
    n_old = int(pre["n_entries"][b])
    kv_rows = list(kv_new) + list(extra_kv)
    n_have = n_old + len(kv_rows)
    E_cap = max(pre["E_cap"], n_have + 1)
    g = {k: pre[k] for k in ("kind", "H", "c", "m", "n_win", "overlap", "vis", "scale",
                             "kv_dtype", "k", "idx_dtype", "sink", "bias_a", "bias_b")}
    act = "bf16" if kvk == "fp8bf16" else kvk  # activations' storage
    g["score_dtype"] = pre.get("score_dtype", "f32")
    for k_ in ("norm_rope", "q_norm_w", "kv_norm_w", "rope_inv_freq", "rope_dims", "norm_eps"):
        if k_ in pre:
            g[k_] = pre[k_]
    g.update(B=1, E_cap=E_cap)
    g["pos"] = np.array([t], dtype=np.int64)
    g["n_entries"] = np.array([n_have], dtype=np.int32)
    kv = np.zeros((1, E_cap, pre["kv_cache"].shape[-1]), dtype=pre["kv_cache"].dtype)
    kv[0, :n_old] = pre["kv_cache"][b, :n_old]
    if kvk == "fp8bf16":
        ks = np.ones((1, E_cap), np.float32)
        ks[0, :n_old] = pre["kv_scale"][b, :n_old]
        if kv_rows:
            kv[0, n_old:n_have], ks[0, n_old:n_have] = fp8bf16_codes_of(np.array(kv_rows))
        g["kv_scale"] = ks
    elif kv_rows:
        kv[0, n_old:n_have] = _bits(np.array(kv_rows), kvk)
    g["kv_cache"] = kv
    tail_len = 2 * m if pre["overlap"] else m
    g["tail_pos0"] = np.array([t - tail_len], dtype=np.int64)
    lo, hi = t - tail_len - pos0, t - pos0
    assert lo >= 0, "tail reaches before the chunk"
    sl = slice(b, b + 1)
    streams = ("ca", "za", "cb", "zb") if pre["overlap"] else ("ca", "za")
    for s in streams:
        g["tail_" + s] = pre[s][sl, lo:hi]
        g["new_" + s] = pre[s][sl, hi]
    w0 = t - (n_win - 1) - (pos0 - (n_win - 1))
    g["win_hist"] = pre["win"][sl, w0:w0 + n_win - 1]
    if pre.get("norm_rope"):
        # the ring holds the history rows prepared at their positions, as stored
        from oracle import position as P
        from oracle.csa import store_as
        from oracle.formats import Stored
        raw = Stored(g["win_hist"][0], act).all()
        hp = np.arange(t - (n_win - 1), t)
        prep = store_as(P.prepare(raw, pre["kv_norm_w"], pre["norm_eps"], hp, pre["rope_inv_freq"]), act)
        g["win_hist"] = _bits(prep, act)[None]
    g["x_new"] = pre["win"][sl, w0 + n_win - 1]
    g["q"] = pre["q"][sl, hi]
    if pre["kind"] == "csa":
        d_I = pre["d_I"]
        g.update(H_I=pre["H_I"], d_I=d_I, ibias_a=pre["ibias_a"], ibias_b=pre["ibias_b"])
        ik = np.zeros((1, E_cap, pre["idx_cache"].shape[-1]), dtype=pre["idx_cache"].dtype)
        ik[0, :n_old] = pre["idx_cache"][b, :n_old]
        idx_rows = list(idx_new) + list(extra_idx)
        g["idx_scale"] = None
        if pre["idx_dtype"] == "e4m3":
            sc = np.ones((1, E_cap), np.float32)
            sc[0, :n_old] = pre["idx_scale"][b, :n_old]
            if idx_rows:
                ik[0, n_old:n_have], sc[0, n_old:n_have] = e4m3_codes_of(np.array(idx_rows))
            g["idx_scale"] = sc
        elif pre["idx_dtype"] == "mxfp4":
            sc = np.zeros((1, E_cap, d_I // 32), np.uint8)
            sc[0, :n_old] = pre["idx_scale"][b, :n_old]
            if idx_rows:
                ik[0, n_old:n_have], sc[0, n_old:n_have] = mxfp4_codes_of(np.array(idx_rows))
            g["idx_scale"] = sc
        elif idx_rows:
            ik[0, n_old:n_have] = _bits(np.array(idx_rows), pre["idx_dtype"])
        g["idx_cache"] = ik
        for s in ("ca", "za", "cb", "zb"):
            g["tail_i" + s] = pre["i" + s][sl, lo:hi]
            g["new_i" + s] = pre["i" + s][sl, hi]
        g["q_idx"] = pre["q_idx"][sl, hi]
        g["q_scale"] = None if pre.get("q_scale") is None else pre["q_scale"][sl, hi]
        g["w_idx"] = pre["w_idx"][sl, hi]
    return g


def varlen_chunk(full, offs, lens, T):
    """A variable-length chunk cut from the aligned prefill workload ``full``
    (whose chunk starts at position full["pos0"]): sequence b's chunk holds
    full's chunk tokens offs[b] .. offs[b] + lens[b] - 1 (seq_pos0 =
    pos0 + offs[b], seq_len = lens[b]) in rows 0 .. lens[b] - 1 of [B][T]
    arrays, the other rows zero; its window rows start n_win - 1 positions
    before the sequence's chunk."""
    g = dict(full)
    B, pos0, n_win = full["B"], int(full["pos0"]), full["n_win"]
    offs = np.asarray(offs, np.int64)
    lens = np.asarray(lens, np.int32)
    g["T"] = T
    g["seq_pos0"] = pos0 + offs
    g["seq_len"] = lens
    for n in ("ca", "za", "cb", "zb", "ica", "iza", "icb", "izb", "q", "q_idx", "w_idx", "q_scale"):
        x = full.get(n)
        if x is None:
            continue
        out = np.zeros((B, T) + x.shape[2:], x.dtype)
        for b in range(B):
            out[b, :lens[b]] = x[b, offs[b]:offs[b] + lens[b]]
        g[n] = out
    W = n_win - 1 + T
    win = np.zeros((B, W) + full["win"].shape[2:], full["win"].dtype)
    for b in range(B):
        n = min(W, full["win"].shape[1] - int(offs[b]))
        win[b, :n] = full["win"][b, offs[b]:offs[b] + n]
    g["win"] = win
    return g
