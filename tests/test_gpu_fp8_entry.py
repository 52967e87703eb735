"""GPU parity of the 576-byte main compressed entry ("DeepSeek-V4" book ch. 8
"The main compressed-entry payload"): the first 448 coordinates as OCP
e4m3fn with one float32 scale per entry, the last 64 (the rotary ones) as
bf16; queries, window rows and token streams stay bf16.  The compressor
and the decode fold store produced entries in this form, and the attention
reads it (the generic kernel decodes each coordinate as it gathers a row).

Rules (tests/compare.py): a produced entry's e4m3 part within one quantum
of the oracle's (a float32 value may sit on a rounding tie), at most 2 % of
codes flipped; its bf16 part, and every output, within the bf16 tolerance.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as OL
from tests.cases import decode_from_prefill, prefix_case
from tests.compare import assert_close, assert_entry_close, check_selection, decode_err, gpu_entries
from tests.test_gpu_parity import _check_decode, _check_prefill, f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("which", ["pro_csa", "flash_hca", "hca_nofold", "csa_norm_rope"])
def test_decode_fp8bf16_entries(gpu_lib, which):
    from sparse_attention_csa_amd.harness import DecodeSession
    if which == "pro_csa":
        g = workloads.pro_csa_decode(seed=141, B=2, n=4 * 3000, H=128, c=512, H_I=64, d_I=128, k=256)
    elif which == "flash_hca":
        g = workloads.flash_hca_decode(seed=142, B=3, n=128 * 300, H=64, c=512)
    elif which == "hca_nofold":
        g = workloads.flash_hca_decode(seed=143, B=2, n=128 * 300, H=64, c=512, pos_off=5)
    else:
        g = workloads.with_norm_rope(workloads.pro_csa_decode(seed=144, B=2, n=4 * 3000, H=128, c=512, H_I=64,
                                                              d_I=128, k=256, idx_dtype="mxfp4"))
    g = workloads.with_fp8bf16_cache(g)
    sess = DecodeSession(g)
    sess.run()
    _check_decode(g, sess, f"fp8bf16-{which}")


def test_prefill_fp8bf16_entries(gpu_lib):
    from sparse_attention_csa_amd.harness import PrefillSession
    a, h = workloads.flash_prefill(seed=145, T=256, n0=1024, H=16, c=512, H_I=8, d_I=32, k=32, m_hca=128)
    for g, label in ((a, "prefill-csa"), (h, "prefill-hca")):
        g = workloads.with_fp8bf16_cache(g)
        sess = PrefillSession(g)
        sess.run()
        _check_prefill(g, sess, f"fp8bf16-{label}")


def test_prefill_then_decode_fp8bf16(gpu_lib):
    """A chunk and then 40 decode steps on the library's own state with the
    576-byte cache: entries the chunk and the steps produce are read back by
    later steps."""
    from sparse_attention_csa_amd.harness import PrefillSession
    from tests.test_gpu_continuation import _stack_steps
    B, n0, T0, steps = 2, 2048, 128, 40
    a, _ = workloads.flash_prefill(seed=146, B=B, T=T0 + steps, n0=n0, H=16, c=512, H_I=64, d_I=128, k=128)
    full = workloads.with_fp8bf16_cache(a)
    pre = prefix_case(full, T0)
    sess = PrefillSession(pre)
    sess.run()
    torch.cuda.synchronize()
    kv_new, idx_new = zip(*[OL.prefill_entries(pre, b) for b in range(B)])
    E0 = int(pre["n_entries"][0])
    for b in range(B):
        assert_entry_close(gpu_entries(sess.state, b, slice(E0, E0 + len(kv_new[b])), "fp8bf16"), kv_new[b],
                           "fp8bf16", f"chunk entries b={b}")
    extra_kv = [[] for _ in range(B)]
    extra_idx = [[] for _ in range(B)]
    E_pre = E0 + T0 // pre["m"]
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
                e = E_pre + len(extra_kv[b])
                assert_entry_close(gpu_entries(sess.state, b, slice(e, e + 1), "fp8bf16"),
                                   np.array(ref["folded_kv"][:1]), "fp8bf16", f"t={t} folded entry b={b}")
                extra_kv[b] += ref["folded_kv"]
                extra_idx[b] += ref["folded_idx"]
            ids = io["topk_idx"][b].cpu().numpy()
            cnt = int(io["topk_cnt"][b])
            ok, swaps, msg = check_selection(ids, cnt, full["k"], ref, decode_err(gs[b], 0, ref))
            assert ok, f"t={t} b={b}: {msg}"
            if swaps:
                ref = OL.decode_step(gs[b], 0, selected=ids[:cnt])
            assert_close(o[b], ref["o"], "bf16", f"t={t} out b={b}")
