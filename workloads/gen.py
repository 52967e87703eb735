"""Seeded generators for the five workloads (and scaled-down variants).

Draw order is fixed per generator; NumPy ``Generator(PCG64(seed))``.  Values
are drawn in float32 and stored as:

* ``"f32"``  float32 arrays;
* ``"bf16"`` uint16 bit patterns, rounded to nearest-even by torch's cast;
* ``"e4m3"`` uint8 OCP e4m3fn codes with one float32 scale per vector
  (scale = max|v| / 448, so nothing saturates), cast by torch.

Dictionary keys follow the layer's vocabulary: ``kv_cache`` (compressed main
entries), ``idx_cache`` (compressed indexer keys), ``tail_*`` (compressor
streams of the tokens whose block is not folded yet, by position from
``tail_pos0``), ``new_*`` (the new token's streams), ``win_hist`` (window rows
before the new token), ``x_new`` (the new token's window row), ``q``,
``q_idx``, ``w_idx``, ``sink``, biases ``bias_*`` / ``ibias_*``.

Stream names: ``ca``/``za`` content and logits of branch a, ``cb``/``zb`` of
branch b; an ``i`` prefix marks the indexer-key streams.
"""

import math

import numpy as np
import torch

CONFIG_NAMES = {
    1: "tiny_csa_f32",
    2: "flash_csa_decode_128k",
    3: "flash_hca_decode_1m",
    4: "pro_csa_decode_1m_fp8idx",
    5: "flash_hybrid_prefill_4096_on_256k",
}

VIS_PRIOR_BLOCKS = 0


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x):
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_rows(x):
    """float32 [..., d] -> (uint8 e4m3fn codes, float32 scale per vector)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def mxfp4_rows(x):
    """float32 [..., d] (d a multiple of 32) -> (packed E2M1 codes [..., d/2]
    uint8, E8M0 block scales [..., d/32] uint8), OCP MX rules: per block of
    32 the scale is 2**(floor(log2 max|v|) - 2), elements v / scale rounded
    to the nearest E2M1 value (ties to the even code), saturating at 6;
    element 2j in the low nibble of byte j."""
    x = np.asarray(x, dtype=np.float64)
    blk = x.reshape(x.shape[:-1] + (-1, 32))
    amax = np.abs(blk).max(axis=-1)
    e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64)
    code = np.where(amax > 0, np.clip(e - 2 + 127, 0, 254), 0).astype(np.uint8)
    y = blk / np.ldexp(1.0, code.astype(np.int64) - 127)[..., None]
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.minimum(np.abs(y), 6.0)
    # nearest grid value; at a midpoint the even code
    idx = np.clip(np.searchsorted(grid, a), 1, 7)
    lo, hi = grid[idx - 1], grid[idx]
    up = (a - lo > hi - a) | ((a - lo == hi - a) & ((idx % 2) == 0))
    mag = np.where(up, idx, idx - 1).astype(np.uint8)
    codes = np.where(np.signbit(y) & (mag > 0), mag | 8, mag).astype(np.uint8).reshape(x.shape)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8), code


def fp8bf16_rows(x):
    """float32 [..., 512] -> (576-byte rows: the first 448 values as e4m3fn
    codes, the last 64 as little-endian bf16; float32 scale per row for the
    e4m3 part, max|v| / 448)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    codes, scale = e4m3_rows(x[..., :448])
    bits = bf16_bits(x[..., 448:])
    out = np.empty(x.shape[:-1] + (576,), np.uint8)
    out[..., :448] = codes
    out[..., 448:] = bits.view(np.uint8).reshape(x.shape[:-1] + (128,))
    return out, scale


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _normal_bf16(rng, shape, chunk_rows=65536):
    """bf16 N(0,1) array, drawn chunk by chunk along the second-to-last axis
    groups (bounded float32 scratch for GiB-sized caches)."""
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        flat[r0:r1] = bf16_bits(_normal(rng, (r1 - r0, shape[-1])))
    return out


def _store(x, kind):
    if kind == "bf16":
        return bf16_bits(x)
    if kind == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# 1. tiny fp32 CSA over a whole 4096-token context
# ---------------------------------------------------------------------------

def tiny_case(seed=0, n=4096, c=64, H=8, H_I=4, d_I=32, k=64, Tq=16, m=4, n_win=128):
    """Context of n tokens x ~ N(0,1) [n][c], compressed at m with one scalar
    logit per token w.x (w ~ N(0, 1/c)); indexer keys from their own raw keys
    x_I ~ N(0,1) [n][d_I] with w_I ~ N(0, 1/d_I); Tq queries at the last Tq
    positions; one sink logit per head."""
    rng = _rng(seed)
    x = _normal(rng, (1, n, c))
    w_cmp = _normal(rng, (c,), 1.0 / math.sqrt(c))
    x_idx = _normal(rng, (1, n, d_I))
    w_cmp_idx = _normal(rng, (d_I,), 1.0 / math.sqrt(d_I))
    q = _normal(rng, (1, Tq, H, c))
    q_idx = _normal(rng, (1, Tq, H_I, d_I))
    w_idx = _normal(rng, (1, Tq, H_I))
    sink = _normal(rng, (H,))
    q_pos = np.arange(n - Tq, n, dtype=np.int64)[None, :]
    return dict(name=CONFIG_NAMES[1], kind="csa", B=1, n=n, c=c, H=H, H_I=H_I, d_I=d_I, k=k,
                Tq=Tq, m=m, n_win=n_win, vis=VIS_PRIOR_BLOCKS, scale=1.0 / math.sqrt(c),
                kv_dtype="f32", idx_dtype="f32", x=x, w_cmp=w_cmp, x_idx=x_idx,
                w_cmp_idx=w_cmp_idx, q=q, q_idx=q_idx, w_idx=w_idx, sink=sink, q_pos=q_pos)


# ---------------------------------------------------------------------------
# decode workloads (one new token per sequence at t = n)
# ---------------------------------------------------------------------------

def _decode_common(rng, kind, B, n, H, c, m, n_win, overlap, kv_dtype, pos_off=0):
    """State and io shared by the CSA and HCA decode workloads.  The new token
    sits at t = n; entries 0 .. n/m-2 are in the cache and the block that
    token n-1 completed is still in the tail, so the step folds it.  With
    0 < pos_off < m the new token sits at t = n + pos_off inside the next
    block instead: all n/m entries are in the cache and the step folds
    nothing (the common decode step)."""
    E = n // m
    tail_len = 2 * m if overlap else m
    g = dict(kind=kind, B=B, n=n, H=H, c=c, m=m, n_win=n_win, overlap=overlap,
             vis=VIS_PRIOR_BLOCKS, scale=1.0 / math.sqrt(c), kv_dtype=kv_dtype, E_cap=E)
    g["pos"] = np.full(B, n + pos_off, dtype=np.int64)
    g["n_entries"] = np.full(B, E - 1 if pos_off == 0 else E, dtype=np.int32)
    g["tail_pos0"] = np.full(B, n + pos_off - tail_len, dtype=np.int64)
    kv = _normal_bf16(rng, (B, E, c)) if kv_dtype == "bf16" else _normal(rng, (B, E, c))
    if pos_off == 0:
        kv[:, E - 1] = 0  # the pending entry is produced by the step
    g["kv_cache"] = kv
    streams = ("ca", "za", "cb", "zb") if overlap else ("ca", "za")
    for s in streams:
        g["tail_" + s] = _store(_normal(rng, (B, tail_len, c)), kv_dtype)
        g["new_" + s] = _store(_normal(rng, (B, c)), kv_dtype)
    g["bias_a"] = _normal(rng, (m, c))
    g["bias_b"] = _normal(rng, (m, c)) if overlap else None
    g["win_hist"] = _store(_normal(rng, (B, n_win - 1, c)), kv_dtype)
    g["x_new"] = _store(_normal(rng, (B, c)), kv_dtype)
    g["q"] = _store(_normal(rng, (B, H, c)), kv_dtype)
    g["sink"] = _normal(rng, (H,))
    return g


def _indexer_state(rng, g, H_I, d_I, k, idx_dtype):
    B, E, m = g["B"], g["E_cap"], g["m"]
    g.update(H_I=H_I, d_I=d_I, k=k, idx_dtype=idx_dtype)
    for s in ("ca", "za", "cb", "zb"):
        g["tail_i" + s] = _store(_normal(rng, (B, 2 * m, d_I)), g["kv_dtype"])
        g["new_i" + s] = _store(_normal(rng, (B, d_I)), g["kv_dtype"])
    g["ibias_a"] = _normal(rng, (m, d_I))
    g["ibias_b"] = _normal(rng, (m, d_I))
    g["w_idx"] = _normal(rng, (B, H_I))


def flash_csa_decode(seed=1, B=8, n=131072, H=64, c=512, H_I=64, d_I=128, k=512, n_win=128,
                     m=4, plant_frac=0.05, plant_gain=3.5):
    """Flash-shaped CSA decode: B sequences of n tokens (n/m entries), bf16.

    Indexer keys ~ N(0,1) except a uniformly random ``plant_frac`` subset P of
    the cached entries per sequence, whose keys get an added component along
    the unit vector u = normalise(sum_h w_h q_h) of that sequence's query:
    K[s] += plant_gain * (1 + z_s / 12) * u, z_s ~ N(0,1).
    This lifts the planted entries' index scores well above the rest (the
    test suite measures the lift with the oracle: about 3 standard deviations)
    without the generator evaluating any score.
    """
    rng = _rng(seed)
    g = _decode_common(rng, "csa", B, n, H, c, m, n_win, True, "bf16")
    g["name"] = CONFIG_NAMES[2]
    _indexer_state(rng, g, H_I, d_I, k, "bf16")
    E = g["E_cap"]
    q_idx = _normal(rng, (B, H_I, d_I))
    g["q_idx"] = bf16_bits(q_idx)
    g["q_scale"] = None
    keys = _normal(rng, (B, E, d_I))
    keys[:, E - 1] = 0
    n_plant = int(round(plant_frac * (E - 1)))
    planted = np.zeros((B, n_plant), dtype=np.int64)
    for b in range(B):
        P = rng.choice(E - 1, size=n_plant, replace=False)
        planted[b] = np.sort(P)
        u = (g["w_idx"][b][:, None] * q_idx[b]).sum(axis=0)
        u = u / np.linalg.norm(u)
        z = rng.standard_normal(n_plant).astype(np.float32)
        amp = np.float32(plant_gain) * (1 + z / 12)
        keys[b, P] += amp[:, None] * u[None, :].astype(np.float32)
    g["idx_cache"] = bf16_bits(keys)
    g["idx_scale"] = None
    g["planted"] = planted
    return g


def pro_csa_decode(seed=3, B=4, n=1 << 20, H=128, c=512, H_I=64, d_I=128, k=1024, n_win=128, m=4,
                   nu=3.0, pos_off=0, idx_dtype="e4m3", score_dtype="f32"):
    """Pro-shaped CSA decode: bf16 KV, fp8 e4m3 indexer queries and keys.

    Indexer keys K[s] = |T_s| z_s with T_s ~ Student-t(nu) and z_s ~ N(0, I),
    which makes the index scores heavy-tailed (the score is positively
    homogeneous in K); keys and queries are stored as e4m3 with one scale per
    vector (per entry for keys, per head for queries).  idx_dtype="mxfp4"
    stores them as OCP MXFP4 instead (E2M1 with one E8M0 scale per block of
    32: the pages' FP4 indexer path), drawn from the same values;
    score_dtype="bf16" selects on bf16-rounded index scores.
    """
    rng = _rng(seed)
    g = _decode_common(rng, "csa", B, n, H, c, m, n_win, True, "bf16", pos_off)
    g["name"] = CONFIG_NAMES[4]
    _indexer_state(rng, g, H_I, d_I, k, idx_dtype)
    g["score_dtype"] = score_dtype
    E = g["E_cap"]
    enc = e4m3_rows if idx_dtype == "e4m3" else mxfp4_rows
    qi = _normal(rng, (B, H_I, d_I))
    g["q_idx"], g["q_scale"] = enc(qi)
    if idx_dtype == "e4m3":
        codes = np.empty((B, E, d_I), dtype=np.uint8)
        scales = np.empty((B, E), dtype=np.float32)
    else:
        codes = np.empty((B, E, d_I // 2), dtype=np.uint8)
        scales = np.empty((B, E, d_I // 32), dtype=np.uint8)
    for b in range(B):
        for s0 in range(0, E, 65536):
            s1 = min(E, s0 + 65536)
            t = np.abs(rng.standard_t(nu, size=s1 - s0)).astype(np.float32)
            z = _normal(rng, (s1 - s0, d_I))
            codes[b, s0:s1], scales[b, s0:s1] = enc(t[:, None] * z)
    if pos_off == 0:
        codes[:, E - 1] = 0
        scales[:, E - 1] = 1 if idx_dtype == "e4m3" else 0
    g["idx_cache"], g["idx_scale"] = codes, scales
    return g


def flash_hca_decode(seed=2, B=8, n=1 << 20, H=64, c=512, n_win=128, m=128, pos_off=0):
    """Flash-shaped HCA decode: n/m entries of dim c, dense attention over all
    of them; the step folds the m-token block that token n-1 completed."""
    rng = _rng(seed)
    g = _decode_common(rng, "hca", B, n, H, c, m, n_win, False, "bf16", pos_off)
    g["name"] = CONFIG_NAMES[3]
    g.update(idx_dtype=None, k=None)
    return g


# ---------------------------------------------------------------------------
# 5. prefill chunk: one CSA layer then one HCA layer
# ---------------------------------------------------------------------------

def _prefill_case(rng, kind, B, T, n0, H, c, m, n_win, overlap, k=None, H_I=None, d_I=None,
                  idx_dtype="bf16"):
    E0 = n0 // m
    E_cap = (n0 + T) // m
    g = dict(kind=kind, B=B, T=T, pos0=n0, H=H, c=c, m=m, n_win=n_win, overlap=overlap,
             vis=VIS_PRIOR_BLOCKS, scale=1.0 / math.sqrt(c), kv_dtype="bf16", E_cap=E_cap, k=k)
    g["n_entries"] = np.full(B, E0, dtype=np.int32)
    kv = np.zeros((B, E_cap, c), dtype=np.uint16)
    kv[:, :E0] = _normal_bf16(rng, (B, E0, c))
    g["kv_cache"] = kv
    streams = ("ca", "za", "cb", "zb") if overlap else ("ca", "za")
    for s in streams:
        g[s] = _normal_bf16(rng, (B, T, c))
    if overlap:
        g["prev_cb"] = _normal_bf16(rng, (B, m, c))
        g["prev_zb"] = _normal_bf16(rng, (B, m, c))
    g["bias_a"] = _normal(rng, (m, c))
    g["bias_b"] = _normal(rng, (m, c)) if overlap else None
    g["win"] = _normal_bf16(rng, (B, n_win - 1 + T, c))
    g["q"] = _normal_bf16(rng, (B, T, H, c))
    g["sink"] = _normal(rng, (H,))
    if kind == "csa":
        g.update(H_I=H_I, d_I=d_I, idx_dtype=idx_dtype, idx_scale=None, q_scale=None)
        if idx_dtype == "e4m3":
            # cached keys and the chunk's indexer queries in e4m3, one scale
            # per vector; entries from E0 on are produced by the chunk
            ik = np.zeros((B, E_cap, d_I), dtype=np.uint8)
            isc = np.ones((B, E_cap), dtype=np.float32)
            ik[:, :E0], isc[:, :E0] = e4m3_rows(_normal(rng, (B, E0, d_I)))
            g["idx_scale"] = isc
        elif idx_dtype == "mxfp4":
            ik = np.zeros((B, E_cap, d_I // 2), dtype=np.uint8)
            isc = np.zeros((B, E_cap, d_I // 32), dtype=np.uint8)
            ik[:, :E0], isc[:, :E0] = mxfp4_rows(_normal(rng, (B, E0, d_I)))
            g["idx_scale"] = isc
        else:
            ik = np.zeros((B, E_cap, d_I), dtype=np.uint16)
            ik[:, :E0] = _normal_bf16(rng, (B, E0, d_I))
        g["idx_cache"] = ik
        for s in ("ca", "za", "cb", "zb"):
            g["i" + s] = _normal_bf16(rng, (B, T, d_I))
        g["prev_icb"] = _normal_bf16(rng, (B, m, d_I))
        g["prev_izb"] = _normal_bf16(rng, (B, m, d_I))
        g["ibias_a"] = _normal(rng, (m, d_I))
        g["ibias_b"] = _normal(rng, (m, d_I))
        if idx_dtype == "e4m3":
            g["q_idx"], g["q_scale"] = e4m3_rows(_normal(rng, (B, T, H_I, d_I)))
        elif idx_dtype == "mxfp4":
            g["q_idx"], g["q_scale"] = mxfp4_rows(_normal(rng, (B, T, H_I, d_I)))
        else:
            g["q_idx"] = _normal_bf16(rng, (B, T, H_I, d_I))
        g["w_idx"] = _normal(rng, (B, T, H_I))
    else:
        g["idx_dtype"] = None
    return g


def flash_prefill(seed=4, B=1, T=4096, n0=262144, H=64, c=512, H_I=64, d_I=128, k=512,
                  n_win=128, m_csa=4, m_hca=128, idx_dtype="bf16"):
    """Flash-shaped hybrid prefill: a T-token chunk appended to an n0-token
    context, through one CSA layer (overlap compressor, indexer, top-k) and one
    HCA layer (non-overlapping compressor, dense), each with its own inputs.
    ``idx_dtype="e4m3"`` stores the CSA indexer keys and queries in e4m3 with
    one scale per vector (the Pro layout)."""
    rng = _rng(seed)
    csa = _prefill_case(rng, "csa", B, T, n0, H, c, m_csa, n_win, True, k, H_I, d_I, idx_dtype)
    hca = _prefill_case(rng, "hca", B, T, n0, H, c, m_hca, n_win, False)
    csa["name"] = CONFIG_NAMES[5] + ":csa"
    hca["name"] = CONFIG_NAMES[5] + ":hca"
    return csa, hca


# ---------------------------------------------------------------------------
# 6. query / KV normalisation and partial rotary positions (any layer case)
# ---------------------------------------------------------------------------

def with_norm_rope(g, seed=7, rope_dims=64, base=10000.0, eps=1e-6):
    """A copy of layer case g with query / KV RMSNorm and partial RoPE on:
    learned scales 1 + 0.1 N(0, 1) (one vector for the query heads, one for
    the KV head), inverse frequencies base^(-2i / rope_dims) as float64,
    epsilon ``eps``.  Drawn from their own generator, so g's other inputs
    are unchanged; g's cached entries and window history stand for vectors
    already prepared."""
    rng = _rng(seed)
    c = g["c"]
    out = dict(g)
    out["norm_rope"] = True
    out["q_norm_w"] = (1.0 + 0.1 * rng.standard_normal(c)).astype(np.float32)
    out["kv_norm_w"] = (1.0 + 0.1 * rng.standard_normal(c)).astype(np.float32)
    out["rope_inv_freq"] = base ** (-np.arange(rope_dims // 2, dtype=np.float64) * 2.0 / rope_dims)
    out["rope_dims"] = rope_dims
    out["norm_eps"] = eps
    return out


def with_fp8bf16_cache(g):
    """A copy of layer case g whose main compressed cache is stored as the
    576-byte FP8 + BF16 entry (the first 448 coordinates e4m3 with one
    float32 scale per entry, the last 64 bf16), re-encoding g's bf16 entries;
    activations stay bf16."""
    out = dict(g)
    kv = np.asarray(g["kv_cache"])
    vals = (kv.astype(np.uint32) << 16).view(np.float32)
    out["kv_cache"], out["kv_scale"] = fp8bf16_rows(vals)
    out["kv_dtype"] = "fp8bf16"
    return out


def block_table(B, n_blocks, seed=11, spare=3):
    """A seeded random block table [B][n_blocks] over a pool of
    B * n_blocks + spare pages (each page owned by one sequence), and the
    pool's page count."""
    rng = _rng(seed)
    n_pages = B * n_blocks + spare
    perm = rng.permutation(n_pages)[:B * n_blocks].astype(np.int32)
    return perm.reshape(B, n_blocks), n_pages


def with_pages(g, page_entries, table=None, n_pages=None, seed=11):
    """A copy of layer case g whose compressed caches live in pages of
    page_entries entries ("DeepSeek-V4" book ch. 13 "Aligning
    original-token blocks": with one 128-token unit per table slot, a CSA
    layer's page holds 32 entries and an HCA layer's one, so one table
    serves both).  The per-sequence caches are padded with empty rows to
    n_blocks * page_entries entries (the capacity the table maps); the
    device state scatters them into a pool of n_pages pages.  Without a
    table, a seeded random one with just enough blocks."""
    out = dict(g)
    B, E = g["B"], g["E_cap"]
    if table is None:
        table, n_pages = block_table(B, -(-E // page_entries), seed)
    table = np.asarray(table, np.int32)
    assert table.shape[0] == B and n_pages is not None
    E_new = table.shape[1] * page_entries
    assert E_new >= E, "the table maps fewer entries than the case holds"
    for name in ("kv_cache", "kv_scale", "idx_cache", "idx_scale"):
        x = g.get(name)
        if x is None:
            continue
        x = np.asarray(x)
        pad = np.zeros((B, E_new - E) + x.shape[2:], x.dtype)
        out[name] = np.concatenate([x, pad], axis=1)
    out.update(E_cap=E_new, page_entries=page_entries, block_table=table, n_pages=n_pages)
    return out
