"""Top-k edge cases through csa_index_topk: exact ties (lower id wins), many
duplicate scores, a threshold bin larger than the in-LDS candidate capacity
(resolution from the score row), fewer visible entries than k, and both
selection modes (split mode for few rows with the MFMA scorer, row mode for
many rows)."""

import numpy as np
import pytest
import torch

from oracle import csa as OC
from oracle.formats import Stored
from tests.compare import score_error_bound, topk_check

pytestmark = pytest.mark.gpu

D = 128


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def _run(keys_f32, q_f32, w, k, n_entries, q_pos, m=4, rows_tq=1):
    from sparse_attention_csa_amd import _lib as L
    B, E, _ = keys_f32.shape
    kb = _bf16(keys_f32).cuda()
    qb = _bf16(q_f32).cuda()
    wt = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    pos = torch.from_numpy(np.asarray(q_pos, np.int64)).cuda()
    ne = torch.from_numpy(np.asarray(n_entries, np.int32)).cuda()
    scores = torch.empty((B, rows_tq, E), dtype=torch.float32, device="cuda")
    ids, cnt = L.csa_index_topk(qb, wt, kb, pos, ne, m, k, scores=scores)
    torch.cuda.synchronize()
    return (kb.view(torch.int16).cpu().numpy().view(np.uint16),
            qb.view(torch.int16).cpu().numpy().view(np.uint16),
            ids.cpu().numpy(), cnt.cpu().numpy())


def _check(kbits, qbits, w, k, n_entries, q_pos, ids, cnt, m=4):
    B, Tq = ids.shape[:2]
    for b in range(B):
        K = Stored(kbits[b], "bf16")
        for t in range(Tq):
            nv = OC.visible_entries(int(q_pos[b][t]), m, int(n_entries[b]))
            q, Kv = Stored(qbits[b, t], "bf16").all(), K.rows(slice(0, nv))
            s = OC.index_scores(q, w[b, t], Kv)
            sel = OC.topk_select(s, k)
            ok, swaps, msg = topk_check(ids[b, t], cnt[b, t], sel, s, k,
                                        err=lambda: score_error_bound(q, w[b, t], Kv))
            assert ok, f"b={b} t={t}: {msg}"


@pytest.mark.parametrize("B,E", [(2, 20000), (1, 4096)])
def test_all_equal_scores_take_lowest_ids(gpu_lib, B, E):
    rng = np.random.default_rng(0)
    v = rng.standard_normal(D).astype(np.float32)
    keys = np.broadcast_to(v, (B, E, D)).copy()
    q = rng.standard_normal((B, 1, 64, D)).astype(np.float32)
    w = np.abs(rng.standard_normal((B, 1, 64))).astype(np.float32)
    k = 512
    pos = np.full((B, 1), 4 * E, np.int64)
    kb, qb, ids, cnt = _run(keys, q, w, k, [E] * B, pos)
    for b in range(B):
        assert cnt[b, 0] == k and np.array_equal(ids[b, 0], np.arange(k))
    _check(kb, qb, w, k, [E] * B, pos, ids, cnt)


def test_many_duplicate_scores(gpu_lib):
    rng = np.random.default_rng(1)
    B, E = 3, 30000
    pool = rng.standard_normal((37, D)).astype(np.float32)
    keys = pool[rng.integers(0, 37, size=(B, E))]
    q = rng.standard_normal((B, 1, 64, D)).astype(np.float32)
    w = rng.standard_normal((B, 1, 64)).astype(np.float32)
    pos = np.full((B, 1), 4 * E, np.int64)
    for k in (1, 100, 1024, 2048):
        kb, qb, ids, cnt = _run(keys, q, w, k, [E] * B, pos)
        _check(kb, qb, w, k, [E] * B, pos, ids, cnt)


def test_threshold_bin_over_capacity(gpu_lib):
    """All scores within 0.1% of each other: 32768 keys share one histogram
    bin, more than the in-LDS candidate capacity."""
    rng = np.random.default_rng(2)
    B, E = 2, 32768
    v = rng.standard_normal(D).astype(np.float32)
    scale = (1.0 + 1e-3 * rng.random((B, E, 1))).astype(np.float32)
    keys = scale * v[None, None, :]
    q = rng.standard_normal((B, 1, 64, D)).astype(np.float32)
    w = np.abs(rng.standard_normal((B, 1, 64))).astype(np.float32)
    pos = np.full((B, 1), 4 * E, np.int64)
    kb, qb, ids, cnt = _run(keys, q, w, 512, [E] * B, pos)
    _check(kb, qb, w, 512, [E] * B, pos, ids, cnt)


def test_fewer_visible_than_k_and_ragged(gpu_lib):
    rng = np.random.default_rng(3)
    B, E = 4, 3000
    keys = rng.standard_normal((B, E, D)).astype(np.float32)
    q = rng.standard_normal((B, 1, 64, D)).astype(np.float32)
    w = rng.standard_normal((B, 1, 64)).astype(np.float32)
    n_entries = [3000, 700, 1, 2999]
    pos = np.array([[4 * 3000], [4 * 800 + 3], [4 * 900], [4 * 513 + 1]], np.int64)
    kb, qb, ids, cnt = _run(keys, q, w, 1024, n_entries, pos)
    _check(kb, qb, w, 1024, n_entries, pos, ids, cnt)
    assert cnt[1, 0] == 700 and cnt[2, 0] == 1 and np.all(ids[2, 0, 1:] == -1)


def test_row_mode_many_queries(gpu_lib):
    """More than 64 query rows: one workgroup per row."""
    rng = np.random.default_rng(4)
    B, Tq, E = 1, 96, 5000
    keys = rng.standard_normal((B, E, D)).astype(np.float32)
    keys[0, 100:400] = keys[0, 50]  # a block of exact duplicates
    q = rng.standard_normal((B, Tq, 64, D)).astype(np.float32)
    w = rng.standard_normal((B, Tq, 64)).astype(np.float32)
    pos = (4 * 4000 + np.arange(Tq) * 9)[None, :].astype(np.int64)
    kb, qb, ids, cnt = _run(keys, q, w, 256, [E], pos, rows_tq=Tq)
    _check(kb, qb, w, 256, [E], pos, ids, cnt)


def _designed_rows(values, Tq=72):
    """Row-mode inputs whose index scores are exactly ``values`` (every row
    the same): one nonzero key coordinate, unit queries, head weights 1/64,
    so each score is max(0, value) summed exactly over the 64 heads."""
    E = values.shape[0]
    keys = np.zeros((1, E, D), np.float32)
    keys[0, :, 0] = values
    q = np.zeros((1, Tq, 64, D), np.float32)
    q[..., 0] = 1.0
    w = np.full((1, Tq, 64), 1.0 / 64, np.float32)
    pos = (4 * E + np.arange(Tq))[None, :].astype(np.int64)
    return keys, q, w, pos


def test_row_mode_threshold_guess_missed(gpu_lib):
    """Row mode guesses the threshold bin from 16 sampled blocks of 256
    scores and reads the row once; here 400 high scores (< k) all sit in the
    sampled blocks, so the guess lies above the row's threshold bin and the
    selection must take its second read of the row."""
    rng = np.random.default_rng(41)
    E, k = 20000, 512
    vals = rng.uniform(0.01, 1.0, E).astype(np.float32)
    starts = [E * b // 16 for b in range(16)]
    hi = np.concatenate([np.arange(s, s + 25) for s in starts])  # 400 positions inside the sample
    vals[hi] = 10.0
    keys, q, w, pos = _designed_rows(vals)
    kb, qb, ids, cnt = _run(keys, q, w, k, [E], pos, rows_tq=q.shape[1])
    _check(kb, qb, w, k, [E], pos, ids, cnt)
    assert np.all(np.isin(hi, ids[0, 0]))


def test_row_mode_stash_overflow(gpu_lib):
    """Row mode with one dominant score value (most of the row in the
    threshold bin): the stash of keys at or above the guessed bin overflows
    and the selection falls back to its second read (ties to lower ids)."""
    rng = np.random.default_rng(42)
    E, k = 20000, 512
    vals = np.full(E, 0.5, np.float32)
    vals[rng.choice(E, 300, replace=False)] = 0.75
    keys, q, w, pos = _designed_rows(vals)
    kb, qb, ids, cnt = _run(keys, q, w, k, [E], pos, rows_tq=q.shape[1])
    _check(kb, qb, w, k, [E], pos, ids, cnt)
