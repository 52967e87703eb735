"""Layer-level pins for the oracle: continuation (prefill then decode equals a
longer prefill on the same tokens, at and across block boundaries), and the
seeded workloads' structure."""

import numpy as np
import pytest

import workloads
from oracle import layer
from tests.cases import decode_from_prefill, prefix_case


def _continuation(pre, T_done, T_full, b=0):
    full = prefix_case(pre, T_full)
    kv_full, idx_full = layer.prefill_entries(full, b)
    part = prefix_case(pre, T_done)
    kv_new, idx_new = layer.prefill_entries(part, b)
    extra_kv, extra_idx = [], []
    pos0 = int(pre["pos0"])
    for i in range(T_done, T_full):
        t = pos0 + i
        dec = decode_from_prefill(pre, T_done, kv_new, idx_new, t, extra_kv, extra_idx, b=b)
        got = layer.decode_step(dec, 0)
        want = layer.prefill_query(full, b, i, kv_full, idx_full)
        assert np.allclose(got["o"], want["o"], rtol=0, atol=1e-12), (pre["kind"], i)
        assert np.allclose(got["lse"], want["lse"], rtol=0, atol=1e-12)
        if pre["kind"] == "csa":
            assert np.array_equal(got["sel"], want["sel"])
        extra_kv += got["folded_kv"]
        extra_idx += got["folded_idx"]
    # entries folded one by one in decode equal those of the longer prefill
    n_part = len(kv_new)
    assert np.array_equal(np.array(extra_kv), kv_full[n_part:n_part + len(extra_kv)])


def test_continuation_csa():
    a, _ = workloads.flash_prefill(seed=21, T=40, n0=64, H=3, c=16, H_I=2, d_I=8, k=6)
    _continuation(a, 32, 40)


def test_continuation_csa_e4m3_indexer_second_sequence():
    """The e4m3 indexer (keys the layer produces are quantised with one scale
    per key, then re-encoded into the decode step's cache) and a sequence
    other than the first of the batch."""
    a, _ = workloads.flash_prefill(seed=23, B=2, T=40, n0=64, H=3, c=16, H_I=2, d_I=8, k=6,
                                   idx_dtype="e4m3")
    _continuation(a, 32, 40, b=1)


def test_continuation_csa_mxfp4_indexer_bf16_scores():
    """The pages' FP4 indexer: keys the layer produces are quantised to
    MXFP4 and re-encoded into the decode step's cache; selection on bf16
    index scores."""
    a, _ = workloads.flash_prefill(seed=24, B=1, T=40, n0=64, H=3, c=16, H_I=2, d_I=64, k=6,
                                   idx_dtype="mxfp4")
    a["score_dtype"] = "bf16"
    _continuation(a, 32, 40)


def test_continuation_hca():
    _, h = workloads.flash_prefill(seed=22, T=512, n0=256, H=2, c=8, m_hca=128, k=4, H_I=2,
                                   d_I=8)
    _continuation(h, 256, 512)


def test_decode_step_folds_exactly_one_pending_block():
    g = workloads.flash_hca_decode(seed=5, B=2, n=1024, H=2, c=8, m=128)
    out = layer.decode_step(g, 1)
    assert len(out["folded_kv"]) == 1
    g = workloads.flash_csa_decode(seed=6, B=2, n=256, H=2, c=8, H_I=2, d_I=8, k=8)
    out = layer.decode_step(g, 0)
    assert len(out["folded_kv"]) == 1 and len(out["folded_idx"]) == 1
    assert len(out["sel"]) == 8 and len(out["scores"]) == 64


def test_workloads_are_deterministic():
    a = workloads.flash_csa_decode(seed=1, B=2, n=512, H=2, c=8, H_I=2, d_I=8, k=8)
    b = workloads.flash_csa_decode(seed=1, B=2, n=512, H=2, c=8, H_I=2, d_I=8, k=8)
    for k, v in a.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(v, b[k]), k


def test_planted_scores_lift_about_three_sigma():
    """The Flash CSA decode workload plants a 5% subset whose index scores sit
    about 3 standard deviations above the rest (measured with the oracle)."""
    from oracle import csa
    from oracle.formats import Stored
    g = workloads.flash_csa_decode(seed=1, B=2, n=4 * 8192)
    for b in range(2):
        K = Stored(g["idx_cache"][b], "bf16").all()[:-1]
        s = csa.index_scores(Stored(g["q_idx"][b], "bf16").all(), g["w_idx"][b], K)
        P = g["planted"][b]
        rest = np.ones(len(s), bool)
        rest[P] = False
        lift = (s[P].mean() - s[rest].mean()) / s[rest].std()
        assert 2.5 < lift < 4.0, lift


@pytest.mark.slow
def test_full_size_shapes():
    g = workloads.flash_hca_decode()
    assert g["kv_cache"].shape == (8, 8192, 512) and g["n_entries"][0] == 8191
    assert g["tail_ca"].shape == (8, 128, 512)
