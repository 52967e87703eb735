"""Byte and FLOP accounting for the hybrid-attention hot path.

Two uses:

* the cost model printed in the "DeepSeek-V4" book, ch. 8 "A Cost Model for
  Long Context" (cache bytes per token, main-attention and indexer FLOPs per
  query), reproduced exactly so the formulas are pinned by the pages;
* the *algorithmic* bytes and FLOPs of one launch of each kernel, which the
  benchmark divides by measured time to report a roofline fraction.
  "Algorithmic" counts only what the method itself must move or compute: the
  indexer-key scan, the gathered top-k rows, the visible HCA entries, the
  window rows, q and o once.  Scratch traffic of an implementation (partials,
  score rows) is not counted.
"""

# MI355X published peaks (dense; no sparsity)
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP32_VALU_TFLOPS = 157.3

DTYPE_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1}


# ---------------------------------------------------------------------------
# cost model of the book, ch. 8
# ---------------------------------------------------------------------------

def gqa_bytes_per_token_layer(kv_heads=8, head_dim=128, bytes_per=2):
    """Separate K and V, per head, per dim: the GQA baseline cache."""
    return 2 * kv_heads * head_dim * bytes_per


def mixed_entry_bytes(fp8_dims=448, bf16_dims=64):
    """One 512-dim entry with 448 FP8 and 64 BF16 (rotary) dims."""
    return fp8_dims * 1 + bf16_dims * 2


def main_bytes_per_token(m, entry_bytes=576):
    return entry_bytes / m


def fp4_indexer_bytes_per_token(d_I=128, m=4):
    return d_I * 0.5 / m


def csa_bytes_per_token(entry_bytes=576, m=4, d_I=128):
    return main_bytes_per_token(m, entry_bytes) + fp4_indexer_bytes_per_token(d_I, m)


def model_cache_bytes(n_tokens, n_csa, n_hca, m=4, m_hca=128):
    return n_tokens * (n_csa * csa_bytes_per_token(m=m) + n_hca * main_bytes_per_token(m_hca))


def attention_flops_per_query(c, E, H):
    """~2cE for the dot products plus ~2cE for the weighted sum, per head."""
    return 4 * c * E * H


def indexer_flops_per_query(H_I, d_I, n_tokens, m=4):
    return 2 * H_I * d_I * n_tokens / m


# ---------------------------------------------------------------------------
# algorithmic bytes / flops of the kernels, per launch
# ---------------------------------------------------------------------------

def vector_bytes(d, dtype):
    """Bytes of one stored vector of d values with its scales: float32 per
    vector for e4m3, one E8M0 byte per 32 values for MXFP4 (d/2 code bytes)."""
    if dtype == "mxfp4":
        return d // 2 + d // 32
    return d * DTYPE_BYTES[dtype] + (4 if dtype == "e4m3" else 0)


def index_scan_bytes(B, Tq, E_vis, H_I, d_I, idx_dtype):
    """Indexer scan: every visible key once (with its scales), the queries
    and head weights once (a fused selection need not write the scores)."""
    keys = B * E_vis * vector_bytes(d_I, idx_dtype)
    q = B * Tq * H_I * (vector_bytes(d_I, idx_dtype) + 4)
    return keys + q


def index_scan_flops(B, Tq, E_vis, H_I, d_I):
    return 2.0 * B * Tq * E_vis * H_I * d_I


def attend_bytes(B, Tq, rows, H, c, kv_dtype="bf16"):
    """Attention: each read row once, q in, o out (+ lse)."""
    kb = DTYPE_BYTES[kv_dtype]
    return B * rows * c * kb + 2 * B * Tq * H * c * kb + B * Tq * H * 4


def attend_flops(B, Tq, rows, H, c):
    return 4.0 * B * Tq * rows * H * c


def fold_bytes(B, m, c, streams, kv_dtype="bf16"):
    """Compressor fold of one block per sequence: the block's source tokens
    (branch a, and branch b of the previous block when overlapping) in, one
    entry out, biases once."""
    kb = DTYPE_BYTES[kv_dtype]
    return B * (streams * m * c * kb + c * kb) + (streams // 2) * m * c * 4


# ---------------------------------------------------------------------------
# a whole layer step
# ---------------------------------------------------------------------------

def decode_layer_bytes(kind, B, E, H, c, n_win, k=None, H_I=None, d_I=None, idx_dtype=None, m=None,
                       overlap=False, kv_dtype="bf16"):
    """Algorithmic HBM bytes of one decode step of a layer (one token per
    sequence, E entries visible): the fold of the completed block, the
    indexer-key scan (CSA), the rows attended (the k selected, or all E, plus
    the window), q in and o out."""
    S = 4 if overlap else 2
    byt = fold_bytes(B, m, c, S, kv_dtype)
    if kind == "csa":
        byt += fold_bytes(B, m, d_I, 4, kv_dtype)
        byt += index_scan_bytes(B, 1, E, H_I, d_I, idx_dtype)
        rows = min(k, E) + n_win
    else:
        rows = E + n_win
    return byt + attend_bytes(B, 1, rows, H, c, kv_dtype)


def prefill_layer_flops(kind, T, pos0, m, H, c, n_win, k=None, H_I=None, d_I=None):
    """Algorithmic FLOPs of a prefill chunk of T queries at positions
    pos0 .. pos0+T-1 (causal): the indexer over each query's visible entries
    (CSA), attention over min(k, visible) (CSA) or all visible (HCA) entries
    plus the window rows."""
    fl = 0.0
    for i in range(T):
        vis = (pos0 + i) // m
        w = min(n_win, pos0 + i + 1)
        if kind == "csa":
            fl += index_scan_flops(1, 1, vis, H_I, d_I)
            fl += attend_flops(1, 1, min(k, vis) + w, H, c)
        else:
            fl += attend_flops(1, 1, vis + w, H, c)
    return fl
