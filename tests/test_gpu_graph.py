"""A layer step captured into a HIP graph (through torch's graph capture: the
library launches on the capturing stream) and replayed: every replay must
equal the eager step bit for bit.  Between replays the program does its own
eager work (restoring the entry counts, a copy, synchronisation), as a
serving loop would.  The library records no memset into the stream: every
counter it needs cleared is returned to zero by its own kernels."""

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _snap(sess):
    r = {n: sess.io[n].detach().clone() for n in ("out", "lse", "topk_idx", "topk_cnt") if n in sess.io}
    r["kv"] = sess.state.kv_cache[:, -1].clone()
    r["n_entries"] = sess.state.n_entries.clone()
    r["win"] = sess.state.win_ring.clone()
    return r


@pytest.mark.parametrize("which", ["pro_csa", "flash_hca", "flash_csa"])
def test_graph_replays_match_eager(gpu_lib, which):
    from sparse_attention_csa_amd.harness import DecodeSession
    if which == "pro_csa":
        g = workloads.pro_csa_decode(seed=111, B=4, n=4 * 30000, H=128, c=512, H_I=64, d_I=128, k=1024)
    elif which == "flash_hca":
        g = workloads.flash_hca_decode(seed=112, B=8, n=128 * 1000, H=64, c=512)
    else:
        g = workloads.flash_csa_decode(seed=113, B=3, n=4 * 5000, H=64, c=512, H_I=64, d_I=128, k=256)
    sess = DecodeSession(g)
    n0 = torch.from_numpy(g["n_entries"]).cuda()
    sess.state.n_entries.copy_(n0)
    sess.run()  # eager (also sets the library's per-device caches)
    torch.cuda.synchronize()
    ref = _snap(sess)
    graph = torch.cuda.CUDAGraph()
    sess.state.n_entries.copy_(n0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        sess.run()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device="cuda")
    for rep in range(5):
        sess.state.n_entries.copy_(n0)
        for n in ("out", "lse"):
            sess.io[n].zero_()
        scratch.normal_()  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = _snap(sess)
        for n in ref:
            assert torch.equal(got[n], ref[n]), f"{which}: replay {rep}: {n} differs from the eager step"
    # eager again after the replays
    sess.state.n_entries.copy_(n0)
    sess.run()
    torch.cuda.synchronize()
    got = _snap(sess)
    for n in ref:
        assert torch.equal(got[n], ref[n]), f"{which}: eager step after replays: {n} differs"
