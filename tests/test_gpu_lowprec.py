"""GPU parity of the pages' low-precision indexer formats ("DeepSeek-V4" book
ch. 16 "The two main FP4 targets", "BF16 index scores"; ch. 8 "The indexer
payload"): MXFP4 indexer queries and keys (E2M1 with one E8M0 scale per 32
values) and index scores rounded to bf16 before the top-k.

* decode, Pro-shaped (128 heads, d_I = 128, 64 indexer heads): the MFMA scan
  with the scaled f8f6f4 product in FP4, the fold workgroup quantising the
  new key to MXFP4, with float32 and with bf16 scores, and e4m3 keys with
  bf16 scores;
* decode with shapes outside the MFMA scan (8 indexer heads, d_I = 64): the
  VALU scorer and the separate fold kernel;
* prefill: the chunk's keys quantised to MXFP4 by the compressor, scored
  by every chunk query;
* csa_index_topk on MXFP4 inputs with bf16 scores, scores compared one by
  one with the oracle's.

Rules (tests/compare.py): produced MXFP4 keys must be one of the roundings
float32 accuracy allows; bf16 selections must be the exact top-k, ties to
the lower id, of scores within the bf16 roundings of the float32 error
intervals."""

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as OL
from oracle.formats import Stored, round_to_bf16
from tests.compare import (ambiguous_mxfp4_keys, assert_close, bf16_score_intervals, check_selection,
                           mxfp4_alternatives, prefill_err, score_bounds, score_error_bound)
from tests.test_gpu_parity import _check_decode, f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx,scores,pos_off", [("mxfp4", "f32", 0), ("mxfp4", "bf16", 0), ("e4m3", "bf16", 0),
                                                ("mxfp4", "bf16", 2)])
def test_decode_pro_low_precision_indexer(gpu_lib, idx, scores, pos_off):
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.pro_csa_decode(seed=121, B=4, n=4 * 20000 + 36, H=128, c=512, H_I=64, d_I=128, k=1024,
                                 idx_dtype=idx, score_dtype=scores, pos_off=pos_off)
    sess = DecodeSession(g)
    sess.run()
    swaps = _check_decode(g, sess, f"pro-{idx}-{scores}-{pos_off}")
    print(f"[pro-{idx}-{scores}] sets differing from the oracle's (within the rules): {swaps}", flush=True)


@pytest.mark.parametrize("scores", ["f32", "bf16"])
def test_decode_mxfp4_valu_scorer(gpu_lib, scores):
    """8 indexer heads of dim 64: the VALU scorer, the separate fold kernel
    and the row-wise top-k."""
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.pro_csa_decode(seed=122, B=2, n=4 * 3000, H=16, c=128, H_I=8, d_I=64, k=128,
                                 idx_dtype="mxfp4", score_dtype=scores)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"valu-mxfp4-{scores}")


@pytest.mark.parametrize("scores", ["f32", "bf16"])
def test_prefill_mxfp4_keys(gpu_lib, scores):
    from sparse_attention_csa_amd.harness import PrefillSession
    g, _ = workloads.flash_prefill(seed=123, T=256, n0=1024, H=16, c=128, H_I=8, d_I=64, k=64,
                                   idx_dtype="mxfp4")
    g["score_dtype"] = scores
    sess = PrefillSession(g)
    sess.run()
    torch.cuda.synchronize()
    kv_new, idx_new, raw = OL.prefill_entries(g, 0, raw=True)
    E0, n_new = int(g["n_entries"][0]), len(kv_new)
    assert int(sess.state.n_entries[0].item()) == E0 + n_new
    assert_close(f64(sess.state.kv_cache[0, E0:E0 + n_new]), kv_new, "bf16", "mxfp4 prefill entries")
    codes = sess.state.idx_cache[0, E0:E0 + n_new].cpu().numpy()
    scl = sess.state.idx_scale[0, E0:E0 + n_new].cpu().numpy()
    got = Stored(codes, "mxfp4", scl).all()
    n_alt = 0
    for i in range(n_new):
        alts = mxfp4_alternatives(raw[i])
        n_alt += len(alts) > 1
        assert any(np.array_equal(got[i], a) for a in alts), f"prefill key {E0 + i}"
    # the GPU's keys, where rounding left a choice, are the ones it scored
    idx_gpu = got
    amb = ambiguous_mxfp4_keys(raw, range(E0, E0 + n_new))
    ids = sess.io["topk_idx"][0].cpu().numpy()
    cnt = sess.io["topk_cnt"][0].cpu().numpy()
    out = f64(sess.io["out"])
    for i in range(g["T"]):
        ref = OL.prefill_query(g, 0, i, kv_new, idx_new)
        bd = {}
        if amb:
            q = Stored(g["q_idx"][0, i], "mxfp4", g["q_scale"][0, i]).all()
            bd = score_bounds(q, np.asarray(g["w_idx"][0, i], np.float64), amb)
        ok, swaps, msg = check_selection(ids[i], cnt[i], g["k"], ref,
                                         prefill_err(g, 0, i, idx_gpu, len(ref["scores"])), bd, scores)
        assert ok, f"mxfp4 prefill q{i}: {msg}"
        if swaps:
            ref = OL.prefill_query(g, 0, i, kv_new, idx_new, selected=ids[i, :cnt[i]])
        assert_close(out[0, i], ref["o"], "bf16", f"mxfp4 prefill out q{i}")
    print(f"[prefill-mxfp4-{scores}] keys with two valid roundings: {n_alt}", flush=True)


@pytest.mark.parametrize("H_I,d_I", [(64, 128), (8, 64)])
def test_index_topk_mxfp4_bf16_scores(gpu_lib, H_I, d_I):
    """csa_index_topk on MXFP4 vectors: every written score within the bf16
    roundings of its float32 error interval, and an exact bf16 top-k."""
    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import dev
    rng = np.random.default_rng(124)
    B, Tq, E, m, k = 3, 1, 5000, 4, 256
    qf = rng.standard_normal((B, Tq, H_I, d_I)).astype(np.float32)
    kf = (np.abs(rng.standard_t(3.0, size=(B, E, 1))) * rng.standard_normal((B, E, d_I))).astype(np.float32)
    qp, qsc = workloads.gen.mxfp4_rows(qf)
    kp, ksc = workloads.gen.mxfp4_rows(kf)
    w = rng.standard_normal((B, Tq, H_I)).astype(np.float32)
    pos = np.array([[4 * E + 3], [4 * 4000 + 1], [4 * 37]], np.int64)
    n_ent = np.array([E, E, E], np.int32)
    scores = torch.full((B, Tq, E), float("nan"), device="cuda")
    ids, cnt = L.csa_index_topk(dev(qp, "u8"), dev(w, "f32"), dev(kp, "u8"), dev(pos, "i64"), dev(n_ent, "i32"),
                                m, k, q_scale=dev(qsc, "u8"), k_scale=dev(ksc, "u8"), scores=scores,
                                idx_dtype=L.CSA_MXFP4, score_bf16=True)
    torch.cuda.synchronize()
    from oracle.csa import index_scores
    from oracle.formats import mxfp4_decode
    for b in range(B):
        nv = int(min(pos[b, 0] // m, E))
        q = mxfp4_decode(qp[b, 0], qsc[b, 0])
        K = mxfp4_decode(kp[b, :nv], ksc[b, :nv])
        raw = index_scores(q, w[b, 0].astype(np.float64), K)
        err = score_error_bound(q, w[b, 0], K)
        lo, hi = bf16_score_intervals(raw, err)
        got = scores[b, 0, :nv].cpu().numpy().astype(np.float64)
        assert np.all((got >= lo) & (got <= hi)), f"b={b}: scores outside their bf16 intervals"
        assert np.array_equal(got, round_to_bf16(got)), f"b={b}: scores not bf16 values"
        ref = {"sel": None, "scores": round_to_bf16(raw), "scores_raw": raw}
        from oracle.csa import topk_select
        ref["sel"] = topk_select(ref["scores"], k)
        ok, _, msg = check_selection(ids[b, 0].cpu().numpy(), int(cnt[b, 0]), k, ref, err, None, "bf16")
        assert ok, f"b={b}: {msg}"
