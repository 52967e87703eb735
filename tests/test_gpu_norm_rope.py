"""GPU parity of the steps on either side of the core attention ("DeepSeek-V4"
book ch. 7 "Query and KV normalization", "Partial rotary position
embeddings", "Why the output is de-rotated"): with norm_rope on, queries and
produced KV vectors (folded entries, window rows) are RMSNorm-ed and their
last 64 coordinates rotated at their positions, and the output's rotary
coordinates are rotated back by the query position.  Compared with the
oracle (oracle/position.py through oracle/layer.py) on the decode paths
(CSA sparse rows, HCA dense MFMA, the generic kernel for other head sizes,
c = 64 where a rotary pair spans two lanes) and on prefill chunks, then a
prefill followed by decode steps on the same state."""

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as OL
from tests.cases import decode_from_prefill, prefix_case
from tests.compare import assert_close, check_selection, decode_err
from tests.test_gpu_parity import _check_decode, _check_prefill, f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("which", ["pro_csa", "flash_hca", "csa_c128", "hca_c64", "csa_e4m3_nofold"])
def test_decode_norm_rope(gpu_lib, which):
    from sparse_attention_csa_amd.harness import DecodeSession
    if which == "pro_csa":
        g = workloads.pro_csa_decode(seed=131, B=3, n=4 * 5000, H=128, c=512, H_I=64, d_I=128, k=512,
                                     idx_dtype="mxfp4")
    elif which == "flash_hca":
        g = workloads.flash_hca_decode(seed=132, B=4, n=128 * 600, H=64, c=512)
    elif which == "csa_c128":
        g = workloads.flash_csa_decode(seed=133, B=2, n=4 * 3000, H=16, c=128, H_I=16, d_I=128, k=256)
    elif which == "hca_c64":
        g = workloads.flash_hca_decode(seed=134, B=2, n=128 * 40, H=8, c=64)
    else:
        g = workloads.pro_csa_decode(seed=135, B=2, n=4 * 3000, H=128, c=512, H_I=64, d_I=128, k=256,
                                     pos_off=2)
    g = workloads.with_norm_rope(g)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"norm-rope-{which}")


@pytest.mark.parametrize("H,c", [(8, 64), (64, 512)])
def test_prefill_norm_rope(gpu_lib, H, c):
    from sparse_attention_csa_amd.harness import PrefillSession
    a, h = workloads.flash_prefill(seed=136, T=256, n0=1024, H=H, c=c, H_I=8, d_I=32, k=32, m_hca=128)
    for g, label in ((workloads.with_norm_rope(a), "prefill-csa"), (workloads.with_norm_rope(h), "prefill-hca")):
        sess = PrefillSession(g)
        sess.run()
        _check_prefill(g, sess, f"norm-rope-{label}-c{c}")


def test_prefill_then_decode_norm_rope(gpu_lib):
    """A chunk then 40 decode steps on the library's own state: the ring
    holds the chunk's prepared window rows, then each step's."""
    from sparse_attention_csa_amd.harness import PrefillSession
    B, n0, T0, steps = 2, 2048, 128, 40
    a, _ = workloads.flash_prefill(seed=137, B=B, T=T0 + steps, n0=n0, H=64, c=512, H_I=64, d_I=128, k=128)
    full = workloads.with_norm_rope(a)
    pre = prefix_case(full, T0)
    sess = PrefillSession(pre)
    sess.run()
    torch.cuda.synchronize()
    kv_new, idx_new = zip(*[OL.prefill_entries(pre, b) for b in range(B)])
    extra_kv = [[] for _ in range(B)]
    extra_idx = [[] for _ in range(B)]
    E_pre = int(pre["n_entries"][0]) + T0 // pre["m"]
    from tests.test_gpu_continuation import _stack_steps
    for j in range(steps):
        t = n0 + T0 + j
        gs = [decode_from_prefill(full, T0, kv_new[b], idx_new[b], t, extra_kv[b], extra_idx[b], b=b)
              for b in range(B)]
        io = sess.decode(_stack_steps(gs))
        torch.cuda.synchronize()
        o = f64(io["out"])
        for b in range(B):
            ref = OL.decode_step(gs[b], 0)
            if ref["folded_kv"]:
                gk = f64(sess.state.kv_cache[b, E_pre + len(extra_kv[b])])
                assert_close(gk[None], np.array(ref["folded_kv"][:1]), "bf16", f"t={t} folded entry b={b}")
                extra_kv[b] += ref["folded_kv"]
                extra_idx[b] += ref["folded_idx"]
            ids = io["topk_idx"][b].cpu().numpy()
            cnt = int(io["topk_cnt"][b])
            ok, swaps, msg = check_selection(ids, cnt, full["k"], ref, decode_err(gs[b], 0, ref))
            assert ok, f"t={t} b={b}: {msg}"
            if swaps:
                ref = OL.decode_step(gs[b], 0, selected=ids[:cnt])
            assert_close(o[b], ref["o"], "bf16", f"t={t} out b={b}")
