"""Run-to-run determinism with the default launch plan (no split_rows): the
same decode step run three times on one state, and the same prefill chunk
run on three fresh copies of one state, give identical bits -- outputs,
lse, top-k ids and counts, entry counts and the entries the step writes
("DeepSeek-V4" book ch. 12 "Batch invariance": bitwise reproducible decode;
no floating-point atomics sit in any result path, and every reduction runs
in a fixed order).  The decode cases are the ones the benchmark times (the
same state stepped again after its entry counts are restored), at a smaller
context; the step is also checked against the oracle once."""

import pytest
import torch

import workloads
from tests.test_gpu_parity import _check_decode

pytestmark = pytest.mark.gpu

DECODE_CASES = {
    "pro_csa_e4m3": lambda: workloads.pro_csa_decode(seed=201, B=4, n=4 * 50000, H=128, c=512, H_I=64, d_I=128,
                                                     k=1024),
    "pro_csa_mxfp4_bf16_scores": lambda: workloads.pro_csa_decode(seed=204, B=4, n=4 * 50000, H=128, c=512,
                                                                  H_I=64, d_I=128, k=1024, idx_dtype="mxfp4",
                                                                  score_dtype="bf16"),
    "flash_csa_bf16": lambda: workloads.flash_csa_decode(seed=202, B=8, n=4 * 16384, H=64, c=512, H_I=64, d_I=128,
                                                         k=512),
    "flash_hca": lambda: workloads.flash_hca_decode(seed=203, B=8, n=128 * 3000, H=64, c=512),
}


def _decode_bits(sess, e0):
    """The step's results: outputs, selection, entry counts, and the cache
    rows at the old entry counts e0 (where a fold writes the new entry, its
    indexer key and their scales)."""
    torch.cuda.synchronize()
    r = {n: sess.io[n].detach().cpu().clone() for n in ("out", "lse", "topk_idx", "topk_cnt") if n in sess.io}
    st = sess.state
    r["n_entries"] = st.n_entries.detach().cpu().clone()
    rows = torch.clamp(e0.long(), max=st.E_cap - 1).to(st.kv_cache.device)
    ar = torch.arange(st.B, device=st.kv_cache.device)
    for name in ("kv_cache", "kv_scale", "idx_cache", "idx_scale"):
        t = getattr(st, name, None)
        if t is not None:
            r[name + "_new"] = t[ar, rows].detach().cpu().clone()
    r["win_ring"] = st.win_ring.detach().cpu().clone()
    return r


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_decode_step_is_bitwise_reproducible(gpu_lib, name):
    from sparse_attention_csa_amd.harness import DecodeSession
    g = DECODE_CASES[name]()
    sess = DecodeSession(g)
    saved = sess.state.n_entries.clone()
    runs = []
    for rep in range(3):
        print(f"[{name}] run {rep}", flush=True)
        sess.state.n_entries.copy_(saved)
        sess.run()
        runs.append(_decode_bits(sess, saved))
    _check_decode(g, sess, f"determinism-{name}")
    for rep in (1, 2):
        for k, v in runs[0].items():
            assert torch.equal(runs[rep][k], v), f"{name}: {k} of run {rep} differs from run 0"


def test_prefill_chunk_is_bitwise_reproducible(gpu_lib):
    from sparse_attention_csa_amd.harness import PrefillSession
    for g in workloads.flash_prefill(seed=205, B=1, T=512, n0=128 * 160, H=64, c=512, H_I=64, d_I=128, k=512):
        runs = []
        for rep in range(3):
            print(f"[prefill {g['kind']}] run {rep}", flush=True)
            sess = PrefillSession(g)
            sess.run()
            torch.cuda.synchronize()
            r = {n: t.detach().cpu().clone() for n, t in sess.io.items()
                 if n in ("out", "lse", "topk_idx", "topk_cnt")}
            st = sess.state
            r["n_entries"] = st.n_entries.detach().cpu().clone()
            r["kv_cache"] = st.kv_cache.detach().cpu().clone()
            r["win_ring"] = st.win_ring.detach().cpu().clone()
            runs.append(r)
            del sess
        for rep in (1, 2):
            for k, v in runs[0].items():
                assert torch.equal(runs[rep][k], v), f"prefill {g['kind']}: {k} of run {rep} differs from run 0"
