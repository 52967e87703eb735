"""Batch invariance of a decode step ("DeepSeek-V4" book ch. 12 "Batch
invariance": a token's output is bitwise unchanged by its placement within
a batch).  With split_rows set in the layer descriptor, every query's rows
are cut into splits of that size whatever the batch; the indexer scores each
key the same way whatever the scan's grid, and the selection is exact.  So a
sequence decoded alone, inside a batch of eight, or at another place of a
smaller batch must give identical bits: output, lse, top-k and the entry the
step folds."""

import numpy as np
import pytest
import torch

import workloads
from tests.test_gpu_parity import _check_decode

pytestmark = pytest.mark.gpu

PER_SEQ = ("pos", "n_entries", "tail_pos0", "kv_cache", "win_hist", "x_new", "q", "q_idx", "q_scale",
           "w_idx", "idx_cache", "idx_scale")


def _select(g, seqs):
    """The decode workload of sequences ``seqs`` of g, in that order."""
    out = dict(g)
    out["B"] = len(seqs)
    for k, v in g.items():
        if v is None or not isinstance(v, np.ndarray):
            continue
        if k in PER_SEQ or k.startswith("tail_") or k.startswith("new_"):
            out[k] = np.ascontiguousarray(v[list(seqs)])
    return out


def _run(g):
    from sparse_attention_csa_amd.harness import DecodeSession
    sess = DecodeSession(g)
    sess.run()
    torch.cuda.synchronize()
    r = {n: sess.io[n].detach().cpu().clone() for n in ("out", "lse", "topk_idx", "topk_cnt") if n in sess.io}
    r["kv"] = sess.state.kv_cache[:, -1].detach().cpu().clone()
    r["n_entries"] = sess.state.n_entries.detach().cpu().clone()
    return sess, r


@pytest.mark.parametrize("which,split", [("pro_csa", 144), ("flash_csa", 160), ("flash_hca", 144),
                                         ("flash_hca_nofold", 272)])
def test_decode_is_batch_invariant(gpu_lib, which, split):
    if which == "pro_csa":
        g = workloads.pro_csa_decode(seed=101, B=8, n=4 * 20000, H=128, c=512, H_I=64, d_I=128, k=1024)
    elif which == "flash_csa":
        g = workloads.flash_csa_decode(seed=102, B=8, n=4 * 8192, H=64, c=512, H_I=64, d_I=128, k=512)
    elif which == "flash_hca":
        g = workloads.flash_hca_decode(seed=103, B=8, n=128 * 2000, H=64, c=512)
    else:
        g = workloads.flash_hca_decode(seed=104, B=8, n=128 * 2000, H=64, c=512, pos_off=17)
    g["split_rows"] = split
    sess, full = _run(g)
    _check_decode(g, sess, f"batch-invariance-{which}-B8")
    del sess
    for seqs in ((3,), (0,), (7,), (5, 3, 1), (6, 2)):
        print(f"[{which}] sequences {seqs}", flush=True)
        _, part = _run(_select(g, seqs))
        for i, b in enumerate(seqs):
            for n in full:
                assert torch.equal(part[n][i], full[n][b]), \
                    f"{which}: {n} of sequence {b} at place {i} of {seqs} differs from place {b} of 8"


def test_split_rows_rejected_beyond_its_limits(gpu_lib):
    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.flash_hca_decode(seed=105, B=2, n=128 * 4000, H=64, c=512)
    g["split_rows"] = 32  # (4000 + 128) / 32 splits > 64
    sess = DecodeSession(g)
    with pytest.raises(L.CsaError, match="split_rows"):
        sess.run()
    g["split_rows"] = 40  # not a multiple of 16
    with pytest.raises(L.CsaError, match="split_rows"):
        DecodeSession(g).run()
