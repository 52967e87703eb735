"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (DecodeSession / PrefillSession through the C ABI).

Decode workloads are checked on every sequence (the oracle scores all visible
entries of a sequence in float64 in a few seconds); the prefill workload is
checked on sampled queries (first, last and spread between, including block
boundaries), with the chunk's compressed entries checked in full."""

import numpy as np
import pytest
import torch

import workloads
from tests.test_gpu_parity import _check_decode, _check_prefill

pytestmark = pytest.mark.gpu


def _run_decode(g, label):
    from sparse_attention_csa_amd.harness import DecodeSession
    print(f"[{label}] upload", flush=True)
    sess = DecodeSession(g)
    sess.run()
    torch.cuda.synchronize()
    print(f"[{label}] compare", flush=True)
    swaps = _check_decode(g, sess, label)
    print(f"[{label}] ok, tie swaps: {swaps}", flush=True)


def test_flash_csa_decode_128k(gpu_lib):
    _run_decode(workloads.flash_csa_decode(), "flash-csa-128k")


def test_flash_hca_decode_1m(gpu_lib):
    _run_decode(workloads.flash_hca_decode(), "flash-hca-1m")


def test_pro_csa_decode_1m_fp8_indexer(gpu_lib):
    _run_decode(workloads.pro_csa_decode(), "pro-csa-1m")


def _all_topk_sets(g, sess, label):
    """Every query's top-k set of the CSA prefill chunk against the oracle's
    selection from its float64 scores (the keys decoded once; queries scored
    in parallel threads, one BLAS thread each)."""
    import concurrent.futures as cf
    import os

    from threadpoolctl import threadpool_limits

    from oracle import csa as OC
    from oracle import layer as OL
    from oracle.formats import Stored
    from tests.compare import score_error_bound, topk_check

    kv_new, idx_new = OL.prefill_entries(g, 0)
    E0 = int(g["n_entries"][0])
    K = np.concatenate([Stored(g["idx_cache"][0], "bf16").rows(slice(0, E0)), idx_new])
    qi = Stored(g["q_idx"][0], "bf16")
    ids = sess.io["topk_idx"][0].cpu().numpy()
    cnt = sess.io["topk_cnt"][0].cpu().numpy()

    def one(i):
        nv = OC.visible_entries(int(g["pos0"]) + i, g["m"], len(K), g["vis"])
        q = qi.rows(i)
        sc = OC.index_scores(q, g["w_idx"][0][i], K[:nv])
        ok, swaps, msg = topk_check(ids[i], cnt[i], OC.topk_select(sc, g["k"]), sc, g["k"],
                                    err=lambda: score_error_bound(q, g["w_idx"][0][i], K[:nv]))
        return i, ok, swaps, msg

    swaps = 0
    with threadpool_limits(1), cf.ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        for i, ok, sw, msg in ex.map(one, range(g["T"])):
            assert ok, f"{label} q{i}: {msg}"
            swaps += sw
            if i % 1024 == 1023:
                print(f"[{label}] top-k sets of queries 0..{i} ok", flush=True)
    return swaps


@pytest.mark.timeout(600)
def test_flash_prefill_4096_on_256k(gpu_lib):
    """Both layers of the prefill chunk.  CSA: every query's top-k set;
    outputs (on the GPU's selection) of 140 queries, every 32nd plus block
    and chunk boundaries.  HCA: outputs of the same queries."""
    from sparse_attention_csa_amd.harness import PrefillSession
    a, h = workloads.flash_prefill()
    T = a["T"]
    sample = sorted(set([0, 1, 3, 4, 127, 128, 1000, 2047, 2048, T - 129, T - 128, T - 2, T - 1] +
                        list(range(5, T, 32))))
    for g, label in ((a, "prefill-csa"), (h, "prefill-hca")):
        print(f"[{label}] upload", flush=True)
        sess = PrefillSession(g)
        sess.run()
        torch.cuda.synchronize()
        if g["kind"] == "csa":
            print(f"[{label}] compare all {T} top-k sets", flush=True)
            swaps = _all_topk_sets(g, sess, label)
            print(f"[{label}] all top-k sets ok, tie swaps: {swaps}", flush=True)
        print(f"[{label}] compare {len(sample)} queries", flush=True)
        _check_prefill(g, sess, label, queries=sample)
        del sess
        torch.cuda.empty_cache()
