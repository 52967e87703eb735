"""hybrid_layer_decode_noalloc (workspace in the library's own device array)
against hybrid_layer_decode with a caller-allocated workspace: the same
inputs in two separate device states, every output compared.  Several calls
in a row on one device, the later ones smaller or of another layer kind, so
the array is reused with other layouts; then the first configuration again."""

import numpy as np
import pytest
import torch

import workloads
from tests.compare import assert_close

pytestmark = pytest.mark.gpu


def _outputs(sess, B):
    st = sess.state
    r = {"out": sess.io["out"], "lse": sess.io["lse"], "n_entries": st.n_entries,
         "kv_last": st.kv_cache[:, -1], "win_ring": st.win_ring, "tail": st.tail}
    if "topk_idx" in sess.io:
        r.update(topk_idx=sess.io["topk_idx"], topk_cnt=sess.io["topk_cnt"], idx_last=st.idx_cache[:, -1])
    return {k: v.detach().cpu().clone() for k, v in r.items()}


def _compare(label, g, ws_sess, na_sess):
    torch.cuda.synchronize()
    a, b = _outputs(ws_sess, g["B"]), _outputs(na_sess, g["B"])
    for k in a:
        if k in ("out", "kv_last"):
            assert_close(b[k].to(torch.float64).numpy(), a[k].to(torch.float64).numpy(), "bf16", f"{label} {k}")
        elif k == "lse":
            assert np.abs(b[k].numpy() - a[k].numpy()).max() < 1e-3, f"{label} lse"
        # the same kernels in the same launch plan: identical bits expected
        assert torch.equal(a[k], b[k]), f"{label}: {k} differs from the workspace entry point"


CASES = [
    ("pro-csa-e4m3-B4", lambda: workloads.pro_csa_decode(seed=91, B=4, n=4 * 60000, H=128, c=512, H_I=64,
                                                          d_I=128, k=1024)),
    ("pro-csa-e4m3-B2-smaller", lambda: workloads.pro_csa_decode(seed=92, B=2, n=4 * 20000, H=128, c=512,
                                                                 H_I=64, d_I=128, k=512)),
    ("flash-hca-B8", lambda: workloads.flash_hca_decode(seed=93, B=8, n=128 * 2000, H=64, c=512)),
    ("flash-hca-B3-smaller-nofold", lambda: workloads.flash_hca_decode(seed=94, B=3, n=128 * 300, H=64, c=512,
                                                                        pos_off=7)),
    ("pro-csa-e4m3-B4-again", lambda: workloads.pro_csa_decode(seed=91, B=4, n=4 * 60000, H=128, c=512, H_I=64,
                                                                d_I=128, k=1024)),
]


def test_noalloc_decode_matches_the_workspace_entry_point(gpu_lib):
    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import DecodeSession
    assert L.lib().hybrid_layer_noalloc_scratch_bytes() == 32 << 20
    for label, make in CASES:
        print(f"[noalloc] {label}", flush=True)
        g = make()
        ws_sess, na_sess = DecodeSession(g), DecodeSession(g)
        ws_sess.run()
        L.hybrid_layer_decode_noalloc(na_sess.desc, na_sess._state_struct, na_sess._io_struct)
        _compare(label, g, ws_sess, na_sess)
        # a second call in a row with the same configuration (no clearing)
        for s in (ws_sess, na_sess):
            s.state.n_entries.copy_(torch.from_numpy(g["n_entries"]).cuda())
        ws_sess.run()
        L.hybrid_layer_decode_noalloc(na_sess.desc, na_sess._state_struct, na_sess._io_struct)
        _compare(label + " (repeat)", g, ws_sess, na_sess)
        del ws_sess, na_sess
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_configuration_beyond_its_array(gpu_lib):
    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import DecodeSession
    g = workloads.pro_csa_decode(seed=95, B=4, n=4 * 3000, H=128, c=512, H_I=64, d_I=128, k=1024)
    sess = DecodeSession(g)
    st = sess._state_struct
    st.E_cap = 1 << 19  # the workspace of 4 x 524,288 entries exceeds 32 MiB
    with pytest.raises(L.CsaError, match="scratch"):
        L.hybrid_layer_decode_noalloc(sess.desc, st, sess._io_struct)
